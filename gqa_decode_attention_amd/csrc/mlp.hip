// The rest of a decoder layer and the model head on gfx950.
//
// Decoder layer: post-attention RMSNorm, the gated SiLU MLP and the residual
// ("Qwen3-ASR -- Latency & Bottleneck Analysis", section 03: the decoder MLP is
// 27.5% of decode and memory-bound at 529 MB/token; section 07 "Norms are real
// money at this size").
//
// Two stream-ordered kernels:
//   k_mlp_up    y = h * g_post / sqrt(mean(h^2) + eps) for the block's 16 rows,
//               formed in registers from the h slice each lane loads as its
//               operand (the rows' sums of squares exchanged through LDS), as
//               two 16-bit terms (hi = rne(y), lo = rne(y - hi)); gate = W_gate y
//               and up = W_up y on v_mfma_f32_16x16x32 (W exact 16-bit);
//               act = silu(gate) * up, stored as hi / lo tiles [2][I / 32][rows][32]
//   k_mlp_down  out = h + W_down act (act as hi + lo)
// A block owns 16 output features x 16 rows; its 8 waves split the
// contraction, request every operand of a batch before the products, and add
// their partial tiles in LDS.  Blocks of one feature tile sit on one XCD.
// (k_mlp_norm, the same normalisation as its own pass into the operand tiling
// [2][H / 32][rows][32], serves the model head.)
#include <hip/hip_ext.h>

#include "device_common.h"
#include "internal.h"

namespace asr {

namespace {

constexpr int kMlpWaves = 8;
constexpr int kMlpBatch = 4;   // 32-wide contraction steps per operand batch
constexpr int kDownBatch = 12; // steps per batch of the down projection (a wave's whole share at intermediate 3072)

struct MlpTile {
  int col, row;
};
__device__ __forceinline__ MlpTile mlp_tile(int b, int rtiles) {
  const int q = b / (8 * rtiles), rem = b - q * 8 * rtiles;
  return MlpTile{q * 8 + rem % 8, rem / 8};
}

// operand-tiled index of (row n, column c) in a [H / 32][rows][32] plane
__device__ __forceinline__ size_t tiled(int c, int n, int rows) { return ((size_t)(c / 32) * rows + n) * 32 + c % 32; }

template <int DT>
__device__ __forceinline__ float load_h(const MlpArgs &A, size_t i) {
  return A.in_f32 ? reinterpret_cast<const float *>(A.h)[i] : cvt16<DT>(reinterpret_cast<const uint16_t *>(A.h)[i]);
}

template <int DT>
__global__ __launch_bounds__(256) void k_mlp_norm(MlpArgs A) {
  __shared__ float s_sum[4];
  const int n = blockIdx.x;
  const int wave = wave_id(), lane = lane_id();
  float ss = 0.f;
  for (int c = threadIdx.x; c < A.H; c += 256) {
    const float v = load_h<DT>(A, (size_t)n * A.H + c);
    ss += v * v;
  }
  ss = wave_sum(ss);
  if (lane == 0) s_sum[wave] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3]) / (float)A.H + A.eps);
  const size_t plane = (size_t)A.H * A.rows;
  for (int c = threadIdx.x; c < A.H; c += 256) {
    const float y = load_h<DT>(A, (size_t)n * A.H + c) * cvt16<DT>(A.g_post[c]) * inv;
    const uint16_t hi = rne16<DT>(y);
    const size_t i = tiled(c, n, A.rows);
    A.y_hl[i] = hi;
    A.y_hl[plane + i] = rne16<DT>(y - cvt16<DT>(hi));
  }
}

// The wave's products over its share [k0, k0 + 32 kw) of the contraction for 16
// weight rows o0 .. o0 + 15 (B operand: the hi / lo tiles of `hl`, planes of K x rows, at row n)
// with W read as whole 128-byte lines: a matrix-core A operand load covers 64
// bytes of 16 rows, and with the streaming hint (which keeps the 311 MB of the
// model head out of the memory-side cache) the line need not be kept for its
// other half (FETCH_SIZE per head call: 531 MB for 311 MB of weights with
// operand-layout loads, 475 MB with whole lines).  Per batch of BATCH
// steps each instruction loads 64 consecutive 16-byte chunks of the batch's
// rows (4 BATCH chunks per row, a multiple of 8: whole lines when the share
// starts on a line), the rows go through the wave's LDS region (chunk c
// of row r at c ^ (r & 15): both the stores and the operand reads are free of
// bank conflicts), and the A operands are read back in the MFMA layout.
// lds: the wave's BATCH x 1 KB.
template <int DT, int BATCH>
__device__ __forceinline__ void line_products(const uint16_t *w, int K, const uint16_t *hl, int rows, int o0, int n,
                                              int k0, int kw, unsigned char *lds, f32x4_t &acc) {
  constexpr int CPR = BATCH * 4;   // 16-byte chunks per row and batch
  static_assert(64 % CPR == 0 || CPR % 8 == 0, "whole lines per load instruction");
  const int lane = lane_id(), i16 = lane % 16, g4 = lane / 16;
  const size_t plane = (size_t)K * rows;
  for (int s0 = 0; s0 < kw; s0 += BATCH) {
    uint4 wa[BATCH], hi[BATCH], lo[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {   // instruction j: chunks f = 64 j + lane, row f / CPR
      const int f = j * 64 + lane, r = f / CPR, c = f % CPR;
      const int col = k0 + min(s0 + c / 4, kw - 1) * 32 + (c % 4) * 8;   // past the share: a repeated step
      wa[j] = ld16_stream(w + (size_t)(o0 + r) * K + col);
    }
#pragma unroll
    for (int s = 0; s < BATCH; ++s) {
      const int kk = k0 + min(s0 + s, kw - 1) * 32;
      const size_t bi = ((size_t)(kk / 32) * rows + n) * 32 + g4 * 8;
      hi[s] = ld16(hl + bi);
      lo[s] = ld16(hl + plane + bi);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch is issued before any use
    wave_lds_sync();                     // the previous batch's operand reads are done
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int f = j * 64 + lane, r = f / CPR, c = f % CPR;
      *reinterpret_cast<uint4 *>(lds + r * CPR * 16 + ((c ^ (r & 15)) << 4)) = wa[j];
    }
    wave_lds_sync();                     // the rows are stored before any lane reads the operand layout
#pragma unroll
    for (int s = 0; s < BATCH; ++s)
      wa[s] = *reinterpret_cast<const uint4 *>(lds + i16 * CPR * 16 + (((s * 4 + g4) ^ i16) << 4));
#pragma unroll
    for (int s = 0; s < BATCH; ++s) {
      if (s0 + s < kw) {
        acc = mfma16x16x32<DT>(wa[s], hi[s], acc);
        acc = mfma16x16x32<DT>(wa[s], lo[s], acc);
      }
    }
  }
}

// KW: 32-wide contraction steps per wave (H / 32 / 8: 4 at hidden 1024, 8 at 2048)
// LS (calls of at most 16 rows): the weight rows as whole lines through LDS; with more rows the
// blocks of a feature tile share its lines in L2 and the 64-128 KB of LDS would cost occupancy
template <int DT, int KW, bool LS>
__global__ __launch_bounds__(kMlpWaves * 64) void k_mlp_up(MlpArgs A) {
  __shared__ f32x4_t s_c[2][kMlpWaves][kWave];
  __shared__ float s_ss[kMlpWaves][16];
  const int wave = wave_id(), lane = lane_id();
  const int i16 = lane % 16, g4 = lane / 16;
  const int rtiles = (A.rows + 15) / 16;
  const MlpTile tm = mlp_tile(blockIdx.x, rtiles);
  const int o0 = tm.col * 16, nb = tm.row * 16;
  const int n = min(nb + i16, A.rows - 1);   // rows past the call repeat the last (not stored)
  const int kw0 = wave * KW * 32;            // the wave's share of the contraction: columns kw0 ..
  const int k0 = kw0 + g4 * 8;               // this lane's 8 columns of each step: k0 + 32 s ..
  // every load before any wait: the gate and up rows o0 .. o0 + 15 of the wave's share (LS:
  // instruction j takes 16-byte chunks 64 j .. 64 j + 63, row f / CPR, chunk f % CPR: whole
  // 128-byte lines when CPR is a multiple of 8), then the lane's slice of row n of h and the
  // post-norm gains of the same columns
  constexpr int CPR = KW * 4;   // 16-byte chunks per row of the share
  uint4 wa[2][KW], gv[KW];
  float hv[KW][8];
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    if constexpr (LS) {
      const int f = j * 64 + lane, r = f / CPR, c = f % CPR;
      wa[0][j] = ld16_stream(A.w_gate + (size_t)(o0 + r) * A.H + kw0 + c * 8);
      wa[1][j] = ld16_stream(A.w_up + (size_t)(o0 + r) * A.H + kw0 + c * 8);
    } else {   // the operand layout directly: row i16, columns k0 + 32 j ..
      wa[0][j] = ld16_stream(A.w_gate + (size_t)(o0 + i16) * A.H + k0 + 32 * j);
      wa[1][j] = ld16_stream(A.w_up + (size_t)(o0 + i16) * A.H + k0 + 32 * j);
    }
  }
#pragma unroll
  for (int st = 0; st < KW; ++st) {
    const size_t i = (size_t)n * A.H + k0 + 32 * st;
    if (A.in_f32) {
      const float4 a = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(A.h) + i);
      const float4 b = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(A.h) + i + 4);
      hv[st][0] = a.x; hv[st][1] = a.y; hv[st][2] = a.z; hv[st][3] = a.w;
      hv[st][4] = b.x; hv[st][5] = b.y; hv[st][6] = b.z; hv[st][7] = b.w;
    } else {
      unpack8<DT>(ld16(reinterpret_cast<const uint16_t *>(A.h) + i), hv[st]);
    }
    gv[st] = ld16(A.g_post + k0 + 32 * st);
  }
  // the weight rows through the wave's LDS (chunk c of row r at c ^ (r & 15)) into the
  // matrix-core operand layout (lane: row i16, chunk 4 s + g4 of step s)
  if constexpr (LS) {
    extern __shared__ __align__(16) unsigned char dyn[];
    unsigned char *lw = dyn + wave * 2 * KW * 1024;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        const int f = j * 64 + lane, r = f / CPR, c = f % CPR;
        *reinterpret_cast<uint4 *>(lw + m * KW * 1024 + r * CPR * 16 + ((c ^ (r & 15)) << 4)) = wa[m][j];
      }
    wave_lds_sync();   // the rows are stored before any lane reads the operand layout
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int st = 0; st < KW; ++st)
        wa[m][st] = *reinterpret_cast<const uint4 *>(lw + m * KW * 1024 + i16 * CPR * 16 + (((st * 4 + g4) ^ i16) << 4));
  }
  // the row's sum of squares: this lane's slice, the 4 lanes of row n, then the 8 waves
  float ss = 0.f;
#pragma unroll
  for (int st = 0; st < KW; ++st)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += hv[st][e] * hv[st][e];
  ss = xsum<16>(ss);
  ss = xsum<32>(ss);
  if (g4 == 0) s_ss[wave][i16] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int wv = 0; wv < kMlpWaves; ++wv) tot += s_ss[wv][i16];
  const float inv = 1.0f / sqrtf(tot / (float)A.H + A.eps);
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int st = 0; st < KW; ++st) {
    float gf[8], y[8];
    unpack8<DT>(gv[st], gf);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = hv[st][e] * gf[e] * inv;
    uint4 hi, lo;
    split8<DT>(y, hi, lo);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      acc[m] = mfma16x16x32<DT>(wa[m][st], hi, acc[m]);
      acc[m] = mfma16x16x32<DT>(wa[m][st], lo, acc[m]);
    }
  }
  s_c[0][wave][lane] = acc[0];
  s_c[1][wave][lane] = acc[1];
  __syncthreads();
  if (wave == 0) {
    f32x4_t gsum = s_c[0][0][lane], usum = s_c[1][0][lane];
#pragma unroll
    for (int wv = 1; wv < kMlpWaves; ++wv) {
      const f32x4_t a = s_c[0][wv][lane], b = s_c[1][wv][lane];
      gsum[0] += a[0]; gsum[1] += a[1]; gsum[2] += a[2]; gsum[3] += a[3];
      usum[0] += b[0]; usum[1] += b[1]; usum[2] += b[2]; usum[3] += b[3];
    }
    const int row = nb + i16;
    if (row < A.rows) {
      uint16_t hv16[4], lv16[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gt = gsum[j];
        const float act = gt / (1.f + __expf(-gt)) * usum[j];
        hv16[j] = rne16<DT>(act);
        lv16[j] = rne16<DT>(act - cvt16<DT>(hv16[j]));
      }
      // features o0 + 4 g4 .. + 3 of the row: adjacent in the tiling
      const size_t i = tiled(o0 + 4 * g4, row, A.rows), plane = (size_t)A.I * A.rows;
      *reinterpret_cast<uint2 *>(A.a_hl + i) =
          make_uint2((uint32_t)hv16[0] | ((uint32_t)hv16[1] << 16), (uint32_t)hv16[2] | ((uint32_t)hv16[3] << 16));
      *reinterpret_cast<uint2 *>(A.a_hl + plane + i) =
          make_uint2((uint32_t)lv16[0] | ((uint32_t)lv16[1] << 16), (uint32_t)lv16[2] | ((uint32_t)lv16[3] << 16));
    }
  }
}

template <int DT>
__global__ __launch_bounds__(kMlpWaves * 64) void k_mlp_down(MlpArgs A) {
  __shared__ f32x4_t s_c[kMlpWaves][kWave];
  const int wave = wave_id(), lane = lane_id();
  const int i16 = lane % 16, g4 = lane / 16;
  const int rtiles = (A.rows + 15) / 16;
  const MlpTile tm = mlp_tile(blockIdx.x, rtiles);
  const int o0 = tm.col * 16, nb = tm.row * 16;
  const int n = nb + i16;
  // the residual, requested before the products
  float res[4] = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0 && n < A.rows) {
#pragma unroll
    for (int j = 0; j < 4; ++j) res[j] = load_h<DT>(A, (size_t)n * A.H + o0 + 4 * g4 + j);
  }
  const int kw = A.I / 32 / kMlpWaves;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // batches of 12 steps (the whole share at intermediate 3072, one wait per batch),
  // W_down as whole lines through the wave's 12 KB of dynamic LDS
  extern __shared__ __align__(16) unsigned char dyn[];
  line_products<DT, kDownBatch>(A.w_down, A.I, A.a_hl, A.rows, o0, min(n, A.rows - 1), wave * kw * 32, kw,
                                dyn + wave * kDownBatch * 1024, acc);
  s_c[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && n < A.rows) {
    f32x4_t c = s_c[0][lane];
#pragma unroll
    for (int wv = 1; wv < kMlpWaves; ++wv) {
      const f32x4_t d = s_c[wv][lane];
      c[0] += d[0]; c[1] += d[1]; c[2] += d[2]; c[3] += d[3];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t o = (size_t)n * A.H + o0 + 4 * g4 + j;
      const float val = c[j] + res[j];
      if (A.out_f32) reinterpret_cast<float *>(A.out)[o] = val;
      else reinterpret_cast<uint16_t *>(A.out)[o] = rne16<DT>(val);
    }
  }
}

// ---------------------------------------------------------------- a few rows on the vector units
//
// With at most kVectorRows rows the MLP is two GEMVs that stream the weights
// once; the matrix-core tiles above would keep 192 and 64 blocks busy at
// hidden 1024 and leave most CUs idle.  Here each wave owns one intermediate
// feature (up: its gate and up rows) or one output feature (down); lane l
// covers input columns (v * 64 + l) * 8 .. + 7, so every wave-wide load reads
// 1 KB contiguously, and every load of a batch is requested before its first
// wait.  act = silu(gate) * up travels in fp32 through the workspace (the
// bytes of the hi / lo tiles of the many-row path).  R: the rows the kernel is
// built for (1, or kVectorRows with the rows past the call skipped).

// columns (v * 64 + lane) * 8 .. + 7 of a row of length len (zeros past it)
template <int DT>
__device__ __forceinline__ void load8(const uint16_t *row, int len, int v, float (&f)[8]) {
  const int c = (v * 64 + lane_id()) * 8;
  if (c < len) {
    unpack8<DT>(ld16(row + c), f);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 0.f;
  }
}

template <int DT, int KV, int R>   // KV = ceil(H / 512)
__global__ __launch_bounds__(256) void k_mlp_up_few(MlpArgs A) {
  const int lane = lane_id();
  const int f = blockIdx.x * 4 + wave_id();   // intermediate feature
  const int H = A.H;
  // every load first: the gate and up rows of f, the post-norm gain, the rows of h
  uint4 wg[KV], wu[KV], gq[KV];
#pragma unroll
  for (int v = 0; v < KV; ++v) {
    const int c = min((v * 64 + lane) * 8, H - 8);
    wg[v] = ld16_stream(A.w_gate + (size_t)f * H + c);
    wu[v] = ld16_stream(A.w_up + (size_t)f * H + c);
    gq[v] = ld16(A.g_post + c);
  }
  float hv[R][KV * 8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = min(r, A.rows - 1);
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int c = (v * 64 + lane) * 8;
      const int cc = min(c, H - 8);
      float *x = hv[r] + v * 8;
      if (A.in_f32) {
        const float *src = reinterpret_cast<const float *>(A.h) + (size_t)n * H + cc;
        const float4 a = *reinterpret_cast<const float4 *>(src), b = *reinterpret_cast<const float4 *>(src + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      } else {
        unpack8<DT>(ld16(reinterpret_cast<const uint16_t *>(A.h) + (size_t)n * H + cc), x);
      }
      if (c >= H) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
    }
  }
  float gf[KV * 8], wgf[KV * 8], wuf[KV * 8];
#pragma unroll
  for (int v = 0; v < KV; ++v) {
    const bool in = (v * 64 + lane) * 8 < H;
    unpack8<DT>(gq[v], gf + v * 8);
    unpack8<DT>(wg[v], wgf + v * 8);
    unpack8<DT>(wu[v], wuf + v * 8);
    if (!in) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wgf[v * 8 + e] = wuf[v * 8 + e] = 0.f;
    }
  }
  float ag[R], au[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    ag[r] = au[r] = 0.f;
    if (r < A.rows) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < KV * 8; ++e) ss += hv[r][e] * hv[r][e];
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)H + A.eps);
#pragma unroll
      for (int e = 0; e < KV * 8; ++e) {
        const float y = hv[r][e] * gf[e] * inv;
        ag[r] += wgf[e] * y;
        au[r] += wuf[e] * y;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < A.rows) {
      ag[r] = wave_sum(ag[r]);
      au[r] = wave_sum(au[r]);
    }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < A.rows) reinterpret_cast<float *>(A.a_hl)[(size_t)r * A.I + f] = ag[r] / (1.f + __expf(-ag[r])) * au[r];
  }
}

template <int DT, int R>
__global__ __launch_bounds__(256) void k_mlp_down_few(MlpArgs A) {
  constexpr int BK = R == 1 ? 8 : 4;   // 1 KB column groups per batch (registers: W and R act rows)
  const int lane = lane_id();
  const int o = blockIdx.x * 4 + wave_id();   // output feature
  const int I = A.I, KI = (I + 511) / 512;
  const float *act = reinterpret_cast<const float *>(A.a_hl);
  float res = 0.f;   // lane r < rows: the residual of row r
  if (lane < R && lane < A.rows) res = load_h<DT>(A, (size_t)lane * A.H + o);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  for (int v0 = 0; v0 < KI; v0 += BK) {
    uint4 w[BK];
    float4 xa[R][BK][2];
#pragma unroll
    for (int b = 0; b < BK; ++b) {
      const int c = min(((v0 + b) * 64 + lane) * 8, I - 8);
      w[b] = ld16_stream(A.w_down + (size_t)o * I + c);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float *src = act + (size_t)min(r, A.rows - 1) * I + c;
        xa[r][b][0] = *reinterpret_cast<const float4 *>(src);
        xa[r][b][1] = *reinterpret_cast<const float4 *>(src + 4);
      }
    }
#pragma unroll
    for (int b = 0; b < BK; ++b) {
      if (((v0 + b) * 64 + lane) * 8 >= I) continue;   // past the row (and past KI)
      float wf[8];
      unpack8<DT>(w[b], wf);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float x8[8] = {xa[r][b][0].x, xa[r][b][0].y, xa[r][b][0].z, xa[r][b][0].w,
                             xa[r][b][1].x, xa[r][b][1].y, xa[r][b][1].z, xa[r][b][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r] += wf[e] * x8[e];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (r < A.rows) acc[r] = wave_sum(acc[r]);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < A.rows) {
      const float val = acc[r] + readlane(res, r);
      if (lane == 0) {
        const size_t i = (size_t)r * A.H + o;
        if (A.out_f32) reinterpret_cast<float *>(A.out)[i] = val;
        else reinterpret_cast<uint16_t *>(A.out)[i] = rne16<DT>(val);
      }
    }
  }
}

// ---------------------------------------------------------------- model head and verify loop
//
// "Can CTC make Qwen3-ASR faster?", section 11 Phase A: a loop that exposes
// one-token decode and logits; verify_block returns the target's argmax at
// every candidate position; strict greedy acceptance; crop to the committed
// prefix (section 03 "Greedy exactness").

// embedding rows of the token ids (16-bit copies); an id outside the table gives a NaN row
template <int DT>
__global__ __launch_bounds__(256) void k_embed(HeadArgs A) {
  const int n = blockIdx.x;
  const int id = A.ids_in[n];
  const bool ok = id >= 0 && id < A.V;
  const uint16_t nan16 = DT == ASR_BF16 ? 0x7FC0 : 0x7E00;
  for (int c = threadIdx.x * 8; c < A.H; c += 256 * 8) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (ok) v = ld16(A.table + (size_t)id * A.H + c);
    else v.x = v.y = v.z = v.w = (uint32_t)nan16 | ((uint32_t)nan16 << 16);
    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(A.x_out) + (size_t)n * A.H + c) = v;
  }
}

// (value, index) kept by the larger value, then the smaller index; NaN never wins
__device__ __forceinline__ void best_of(float &v, int &i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Logits of 8 vocab tiles of 16 (one per wave) x 16 rows on the matrix cores
// (W_lm exact 16-bit, the normalised rows as hi + lo), and the best (logit,
// id) of each row over the block's 128 ids: partial [block][row].
template <int DT>
__global__ __launch_bounds__(kMlpWaves * 64) void k_head_argmax(HeadArgs A) {
  __shared__ float s_v[kMlpWaves][16];
  __shared__ int s_i[kMlpWaves][16];
  __shared__ __align__(16) unsigned char s_w[kMlpWaves][kMlpBatch * 1024];   // each wave's W rows of a batch
  const int wave = wave_id(), lane = lane_id();
  const int i16 = lane % 16, g4 = lane / 16;
  const int nb = blockIdx.y * 16, n = nb + i16;
  const int v0 = (blockIdx.x * kMlpWaves + wave) * 16;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if (v0 < A.V) {
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    line_products<DT, kMlpBatch>(A.w_lm, A.H, A.y_hl, A.rows, v0, min(n, A.rows - 1), 0, A.H / 32, s_w[wave], acc);
#pragma unroll
    for (int j = 0; j < 4; ++j) best_of(bv, bi, acc[j], v0 + 4 * g4 + j);
  }
  // over the four lane groups of a row (lanes n, n + 16, n + 32, n + 48)
  {
    float v2 = xpart<16>(bv);
    int i2 = __builtin_bit_cast(int, xpart<16>(__builtin_bit_cast(float, bi)));
    best_of(bv, bi, v2, i2);
    v2 = xpart<32>(bv);
    i2 = __builtin_bit_cast(int, xpart<32>(__builtin_bit_cast(float, bi)));
    best_of(bv, bi, v2, i2);
  }
  if (g4 == 0) {
    s_v[wave][i16] = bv;
    s_i[wave][i16] = bi;
  }
  __syncthreads();
  if (threadIdx.x < 16 && nb + (int)threadIdx.x < A.rows) {
    float v = s_v[0][threadIdx.x];
    int i = s_i[0][threadIdx.x];
#pragma unroll
    for (int wv = 1; wv < kMlpWaves; ++wv) best_of(v, i, s_v[wv][threadIdx.x], s_i[wv][threadIdx.x]);
    const size_t p = (size_t)blockIdx.x * A.rows + nb + threadIdx.x;
    A.part_v[p] = v;
    A.part_i[p] = i;
  }
}

// the best of a row's partials: its argmax id (-1 when no logit is a number) and logit
__global__ __launch_bounds__(256) void k_head_reduce(HeadArgs A) {
  __shared__ float s_v[4];
  __shared__ int s_i[4];
  const int n = blockIdx.x, wave = wave_id(), lane = lane_id();
  float v = -INFINITY;
  int i = 0x7fffffff;
  for (int b = threadIdx.x; b < A.nparts; b += 256) best_of(v, i, A.part_v[(size_t)b * A.rows + n], A.part_i[(size_t)b * A.rows + n]);
  for (int m = 32; m >= 1; m >>= 1) {
    const float v2 = __shfl_xor(v, m, kWave);
    const int i2 = __shfl_xor(i, m, kWave);
    best_of(v, i, v2, i2);
  }
  if (lane == 0) {
    s_v[wave] = v;
    s_i[wave] = i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) best_of(v, i, s_v[w], s_i[w]);
    A.ids_out[n] = i == 0x7fffffff ? -1 : i;
    if (A.max_logit) A.max_logit[n] = v;
  }
}

// strict greedy acceptance of each sequence's k drafts against the target's
// argmax of the block rows, then the lengths that keep the committed rows
__global__ __launch_bounds__(256) void k_lens_copy(AcceptArgs A) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s < A.batch_cap) A.new_lens[s] = A.lens[s];
}
__global__ __launch_bounds__(256) void k_accept(AcceptArgs A) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= A.B) return;
  const size_t base = A.qo_n ? (size_t)A.qo[b] : (size_t)b * A.k;
  const int k = A.qo_n ? A.qo[b + 1] - A.qo[b] : A.k;
  const int *d = A.draft + base, *t = A.target + base;
  int a = 0;
  while (a < k && d[a] == t[a]) ++a;
  const int committed = a < k ? a + 1 : k;
  A.accepted[b] = a;
  A.next_token[b] = a < k ? t[a] : d[k - 1];
  const int s = A.slots ? A.slots[b] : b;
  if (s >= 0 && s < A.batch_cap) A.new_lens[s] = max(A.lens[s] - k + committed, 0);
}

using MlpKernel = void (*)(MlpArgs);

hipError_t launch(MlpKernel k, dim3 grid, dim3 block, hipStream_t s, hipEvent_t *ev, int phase, const MlpArgs &a,
                  unsigned lds = 0) {
  if (ev)
    hipExtLaunchKernelGGL(k, grid, block, lds, s, ev[2 * phase], ev[2 * phase + 1], 0u, a);
  else
    hipLaunchKernelGGL(k, grid, block, lds, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t mlp_launch(const MlpArgs &a, hipStream_t s, hipEvent_t *ev) {
  hipError_t e;
  if (a.rows <= kVectorRows) {   // the vector-unit GEMVs: one wave per feature
    const bool one = a.rows == 1;
    MlpKernel up = nullptr;
    switch ((a.H + 511) / 512) {
#define ASR_MLP_UP_FEW(K) \
      case K: up = one ? k_mlp_up_few<DT, K, 1> : k_mlp_up_few<DT, K, kVectorRows>; break;
      ASR_MLP_UP_FEW(1) ASR_MLP_UP_FEW(2) ASR_MLP_UP_FEW(3) ASR_MLP_UP_FEW(4)
#undef ASR_MLP_UP_FEW
      default: return hipErrorInvalidValue;
    }
    if ((e = launch(up, dim3(a.I / 4), dim3(256), s, ev, 0, a)) != hipSuccess) return e;
    return launch(one ? k_mlp_down_few<DT, 1> : k_mlp_down_few<DT, kVectorRows>, dim3(a.H / 4), dim3(256), s, ev, 1, a);
  }
  const int rtiles = (a.rows + 15) / 16;
  const bool ls = rtiles == 1;   // weight lines through LDS for calls of at most 16 rows
  MlpKernel up = nullptr;
  switch (a.H / 32 / kMlpWaves) {
    case 1: up = ls ? k_mlp_up<DT, 1, true> : k_mlp_up<DT, 1, false>; break;
    case 2: up = ls ? k_mlp_up<DT, 2, true> : k_mlp_up<DT, 2, false>; break;
    case 3: up = ls ? k_mlp_up<DT, 3, true> : k_mlp_up<DT, 3, false>; break;
    case 4: up = ls ? k_mlp_up<DT, 4, true> : k_mlp_up<DT, 4, false>; break;
    case 5: up = ls ? k_mlp_up<DT, 5, true> : k_mlp_up<DT, 5, false>; break;
    case 6: up = ls ? k_mlp_up<DT, 6, true> : k_mlp_up<DT, 6, false>; break;
    case 7: up = ls ? k_mlp_up<DT, 7, true> : k_mlp_up<DT, 7, false>; break;
    case 8: up = ls ? k_mlp_up<DT, 8, true> : k_mlp_up<DT, 8, false>; break;
    default: return hipErrorInvalidValue;
  }
  // (dynamic LDS: each wave's gate and up rows of its share, 2 matrices x 16 rows x H / 8 columns
  // x 2 bytes = 8 H bytes per wave; 128 KB at hidden 2048)
  if ((e = launch(up, dim3(a.I / 16 * rtiles), dim3(kMlpWaves * kWave), s, ev, 0, a, ls ? kMlpWaves * 8 * a.H : 0)) !=
      hipSuccess)
    return e;
  return launch(k_mlp_down<DT>, dim3(a.H / 16 * rtiles), dim3(kMlpWaves * kWave), s, ev, 1, a,
                kMlpWaves * kDownBatch * 1024);
}

template <int DT>
hipError_t head_launch(const MlpArgs &norm, const HeadArgs &h, hipStream_t s) {
  hipLaunchKernelGGL(k_mlp_norm<DT>, dim3(norm.rows), dim3(256), 0, s, norm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_head_argmax<DT>, dim3(h.nparts, (h.rows + 15) / 16), dim3(kMlpWaves * kWave), 0, s, h);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_head_reduce, dim3(h.rows), dim3(256), 0, s, h);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mlp(const MlpArgs &a, int dtype, hipStream_t s, hipEvent_t *ev) {
  return dtype == ASR_BF16 ? mlp_launch<ASR_BF16>(a, s, ev) : mlp_launch<ASR_F16>(a, s, ev);
}

hipError_t launch_embed(const HeadArgs &a, int dtype, hipStream_t s) {
  if (dtype == ASR_BF16) hipLaunchKernelGGL(k_embed<ASR_BF16>, dim3(a.rows), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_embed<ASR_F16>, dim3(a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_head(const MlpArgs &norm, const HeadArgs &h, int dtype, hipStream_t s) {
  return dtype == ASR_BF16 ? head_launch<ASR_BF16>(norm, h, s) : head_launch<ASR_F16>(norm, h, s);
}

hipError_t launch_accept(const AcceptArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(k_lens_copy, dim3((a.batch_cap + 255) / 256), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_accept, dim3((a.B + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace asr
