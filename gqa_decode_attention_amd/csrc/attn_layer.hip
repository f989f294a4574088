// One attention-block layer call (decode or k-token verify) on gfx950.
//
// Three phases; every phase is a loop over independent work items, written as
// device functions that both dispatch modes share:
//   A. QKV tiles     input RMSNorm fused into the q/k/v projection (GEMV over rows)
//   C. attention     one item per (row, kv head g, chunk of keys): per-head RMSNorm
//                    and rotary of q (and of the new k rows the chunk holds), KV
//                    append, single-pass online-softmax attention of all q heads of
//                    g over the chunk, a partial (m, l, acc) per q head; the last
//                    item of a (row, g) to finish merges its chunks (log-sum-exp)
//   D. o_proj tiles  output projection (+ residual); lengths advanced
// ASR_DISPATCH_MULTI runs A, C, D as three kernels in stream order.
// ASR_DISPATCH_FUSED runs them in one persistent kernel whose workgroups meet at
// a grid barrier between phases (two per call).
//
// The operation list follows "Qwen3-ASR -- Latency & Bottleneck Analysis",
// section 07 (q/k/v projections, GQA repeat_kv, QK^T, fp32 softmax, AV, o_proj)
// with the norms of "Norms are real money at this size" and the fp32 rotary of
// the section 03 table.  The causal rule of verify rows follows "Can CTC make
// Qwen3-ASR faster?", section 03: position i sees the committed prefix and the
// candidates up to i.
#include "device_common.h"
#include "internal.h"

namespace asr {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr long long kBarrierTimeoutTicks = 50000000;   // wall clock ticks (about 0.5 s at 100 MHz)

struct RowInfo {
  int slot, L, pos, nvis, r;
  bool ok, slot_ok;
};

// Row `row` = (sequence b, block offset r).  Visible keys: L + r + 1.
__device__ __forceinline__ RowInfo row_info(const LayerArgs &A, int row) {
  RowInfo ri;
  const int b = row / A.n;
  ri.r = row - b * A.n;
  const int s = A.slots ? A.slots[b] : b;
  ri.slot = s;
  ri.slot_ok = (s >= 0 && s < A.batch_cap);
  const int L = ri.slot_ok ? A.lens[s] : 0;
  ri.L = L;
  ri.ok = ri.slot_ok && L >= 0 && L + A.n <= A.capacity;
  ri.pos = (A.positions ? A.positions[b] : L) + ri.r;
  ri.nvis = ri.ok ? L + ri.r + 1 : 0;
  return ri;
}

__device__ __forceinline__ int chunks_of(int nvis, int split) { return (nvis + split - 1) / split; }

// rotary angle of pair t at position pos: pos * theta^(-2t/d), formed in fp64
__device__ __forceinline__ void rope_cs(int pos, int t, float theta, float &c, float &s) {
  const double omega = exp2(-(2.0 * t / kHeadDim) * log2((double)theta));
  double sn, cs;
  sincos((double)pos * omega, &sn, &cs);
  c = (float)cs;
  s = (float)sn;
}

// ---------------------------------------------------------------- phase A: QKV projection
//
// Wave w of tile t owns RPW consecutive output rows; their weights stay in
// registers while the wave walks over the input rows RB at a time.  Lane l
// covers columns (v * 64 + l) * 8 .. + 7 for v < KV, so every wave-wide load
// reads 1 KB contiguously.  RMSNorm: h = x * g / sqrt(mean(x^2) + eps).
template <int DT, int KV, int RB, int RPW>
__device__ void qkv_tile(const LayerArgs &A, int tile) {
  const int wave = wave_id(), lane = lane_id();
  const int o0 = (tile * 4 + wave) * RPW;
  const int H = A.H;
  uint4 wr[RPW][KV];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int v = 0; v < KV; ++v)
      wr[i][v] = ld16_stream(A.w_qkv + (size_t)(o0 + i) * H + (v * 64 + lane) * 8);
  float g[KV * 8];
#pragma unroll
  for (int v = 0; v < KV; ++v) unpack8<DT>(ld16(A.g_in + (v * 64 + lane) * 8), g + v * 8);

  for (int rb = 0; rb < A.rows; rb += RB) {
    float x[RB][KV * 8];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = rb + r;
      float ss = 0.f;
      if (row < A.rows) {
#pragma unroll
        for (int v = 0; v < KV; ++v) unpack8<DT>(ld16(A.x + (size_t)row * H + (v * 64 + lane) * 8), x[r] + v * 8);
#pragma unroll
        for (int e = 0; e < KV * 8; ++e) ss += x[r][e] * x[r][e];
      } else {
#pragma unroll
        for (int e = 0; e < KV * 8; ++e) x[r][e] = 0.f;
      }
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)H + A.eps);
#pragma unroll
      for (int e = 0; e < KV * 8; ++e) x[r][e] *= g[e] * inv;
    }
    float acc[RPW][RB];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[i][r] = 0.f;
#pragma unroll
      for (int v = 0; v < KV; ++v) {
        float wf[8];
        unpack8<DT>(wr[i][v], wf);
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][r] += wf[e] * x[r][v * 8 + e];
      }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[i][r] = wave_sum(acc[i][r]);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = rb + r;
      if (row < A.rows && lane < RPW) {
        float val = acc[0][r];
#pragma unroll
        for (int i = 1; i < RPW; ++i)
          if (lane == i) val = acc[i][r];
        A.qkv[(size_t)row * A.nqkv + o0 + lane] = val;
      }
    }
  }
}

// Row table for phase D (which must not read lens: lengths change there).
__device__ void write_row_table(const LayerArgs &A) {
  for (int row = threadIdx.x; row < A.rows; row += blockDim.x) {
    const RowInfo ri = row_info(A, row);
    int4 rec;
    rec.x = ri.ok;
    rec.y = ri.L;
    rec.z = ri.slot;
    rec.w = ri.slot_ok;
    A.rowtab[row] = rec;
  }
}

// ---------------------------------------------------------------- phase C: attention
//
// Items are (row, kv head g, chunk c) for every chunk of `split` keys that holds
// a visible key of the row.  A block-wide prefix sum over the rows' chunk counts
// (from lens, on the device: no host readback) maps a flat item id to its
// (row, g, c).
//
// Lane layout: groups of 8 lanes; a group owns one key row (8 lanes x 16 dims =
// 128 dims, 256 contiguous bytes); a wave takes 8 keys per step, the block 32.
// Each wave keeps a running max and sum per q head (online softmax), so K and
// V stream once with no score buffer; the 4 waves are combined in LDS at the
// end of the item.
template <int GROUP>
struct AttnShared {
  float q[GROUP][kHeadDim];
  float acc[4][GROUP][kHeadDim];
  float m[4][GROUP], l[4][GROUP];
  float mc[GROUP][kMaxChunks], lc[GROUP][kMaxChunks];
  int wsum[4];
  int flag;
};

// block-wide exclusive prefix of (chunks per row) * nkv into pre[0..rows]
__device__ void build_item_prefix(const LayerArgs &A, int *pre, int *wsum) {
  const int wave = wave_id(), lane = lane_id();
  const int rows = A.rows;
  const int per = (rows + 255) / 256;
  const int beg = min((int)threadIdx.x * per, rows), end = min(beg + per, rows);
  int local = 0;
  for (int i = beg; i < end; ++i) local += chunks_of(row_info(A, i).nvis, A.split) * A.nkv;
  int incl = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  int run = base + incl - local;
  for (int i = beg; i < end; ++i) {
    pre[i] = run;
    run += chunks_of(row_info(A, i).nvis, A.split) * A.nkv;
  }
  if (threadIdx.x == 255) pre[rows] = run;
  __syncthreads();
}

// one wave: per-head RMSNorm (gain gp) and rotary of a 128-vector held as the
// pairs (u0, u1) = (t, t + 64) of lane t
template <int DT>
__device__ __forceinline__ void norm_rope(float &u0, float &u1, const uint16_t *gp, float eps, int pos,
                                          float theta, int lane) {
  const float ss = wave_sum(u0 * u0 + u1 * u1);
  const float inv = 1.0f / sqrtf(ss / (float)kHeadDim + eps);
  u0 *= cvt16<DT>(gp[lane]) * inv;
  u1 *= cvt16<DT>(gp[lane + 64]) * inv;
  float c, s;
  rope_cs(pos, lane, theta, c, s);
  const float r0 = u0 * c - u1 * s;
  const float r1 = u1 * c + u0 * s;
  u0 = r0;
  u1 = r1;
}

template <int DT, int GROUP>
__device__ void attn_item(const LayerArgs &A, int item, const int *pre, uint16_t *knew, uint16_t *vnew,
                          AttnShared<GROUP> &S) {
  const int wave = wave_id(), lane = lane_id();
  const int kl = lane & 7, kr = lane >> 3;
  int lo = 0, hi = A.rows;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= item) lo = mid; else hi = mid;
  }
  const int row = lo;
  const int nch = (pre[row + 1] - pre[row]) / A.nkv;
  const int rem = item - pre[row];
  const int g = rem / nch, c = rem - g * nch;
  const RowInfo ri = row_info(A, row);
  const int L = ri.L;
  const int t0 = c * A.split, t1 = min(t0 + A.split, ri.nvis);
  const int nb = max(t0, L);            // first appended position inside the chunk
  const int n_new = max(0, t1 - nb);    // appended rows this chunk sees
  const bool writer = (ri.r == A.n - 1);

  // q of the GROUP heads: norm, rotate, pre-scale by log2(e)/sqrt(d)
  for (int j = wave; j < GROUP; j += 4) {
    const float *src = A.qkv + (size_t)row * A.nqkv + (g * GROUP + j) * kHeadDim;
    float u0 = src[lane], u1 = src[lane + 64];
    norm_rope<DT>(u0, u1, A.g_q, A.eps, ri.pos, A.theta, lane);
    const float qs = kLog2e * rsqrtf((float)kHeadDim);
    S.q[j][lane] = u0 * qs;
    S.q[j][lane + 64] = u1 * qs;
  }
  // new K/V rows at positions nb .. t1-1 (rows r' = p - L of this sequence): rounded
  // as the cache stores them; the last row's item also writes them to the cache
  for (int i = wave; i < n_new; i += 4) {
    const int rp = nb + i - L;
    const int rrow = row - ri.r + rp;
    const float *src = A.qkv + (size_t)rrow * A.nqkv;
    float k0 = src[(A.nq + g) * kHeadDim + lane], k1 = src[(A.nq + g) * kHeadDim + lane + 64];
    norm_rope<DT>(k0, k1, A.g_k, A.eps, ri.pos - ri.r + rp, A.theta, lane);
    const uint16_t kb0 = rne16<DT>(k0), kb1 = rne16<DT>(k1);
    const uint16_t vb0 = rne16<DT>(src[(A.nq + A.nkv + g) * kHeadDim + lane]);
    const uint16_t vb1 = rne16<DT>(src[(A.nq + A.nkv + g) * kHeadDim + lane + 64]);
    knew[i * kHeadDim + lane] = kb0;
    knew[i * kHeadDim + lane + 64] = kb1;
    vnew[i * kHeadDim + lane] = vb0;
    vnew[i * kHeadDim + lane + 64] = vb1;
    if (writer) {
      const size_t off = (((size_t)ri.slot * A.nkv + g) * A.capacity + nb + i) * kHeadDim;
      A.kc[off + lane] = kb0;
      A.kc[off + lane + 64] = kb1;
      A.vc[off + lane] = vb0;
      A.vc[off + lane + 64] = vb1;
    }
  }
  __syncthreads();

  float q[GROUP][16];
#pragma unroll
  for (int j = 0; j < GROUP; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) q[j][e] = S.q[j][kl * 16 + e];

  const size_t kvrow0 = ((size_t)ri.slot * A.nkv + g) * A.capacity;
  const uint16_t *Kp = A.kc + kvrow0 * kHeadDim + kl * 16;
  const uint16_t *Vp = A.vc + kvrow0 * kHeadDim + kl * 16;

  float m[GROUP], l[GROUP], acc[GROUP][16];
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  }
  for (int tb = t0 + wave * 8; tb < t1; tb += 32) {
    const int t = tb + kr;
    const bool valid = t < t1;
    const int tc = valid ? t : t1 - 1;
    uint4 ka, kb, va, vb;
    if (tc < L) {
      ka = ld16_stream(Kp + (size_t)tc * kHeadDim);
      kb = ld16_stream(Kp + (size_t)tc * kHeadDim + 8);
      va = ld16_stream(Vp + (size_t)tc * kHeadDim);
      vb = ld16_stream(Vp + (size_t)tc * kHeadDim + 8);
    } else {
      const uint16_t *kn = knew + (tc - nb) * kHeadDim + kl * 16;
      const uint16_t *vn = vnew + (tc - nb) * kHeadDim + kl * 16;
      ka = *reinterpret_cast<const uint4 *>(kn);
      kb = *reinterpret_cast<const uint4 *>(kn + 8);
      va = *reinterpret_cast<const uint4 *>(vn);
      vb = *reinterpret_cast<const uint4 *>(vn + 8);
    }
    float kf[16], vf[16];
    unpack8<DT>(ka, kf);
    unpack8<DT>(kb, kf + 8);
    unpack8<DT>(va, vf);
    unpack8<DT>(vb, vf + 8);
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) s += q[j][e] * kf[e];
      s = group_sum<8>(s);
      s = valid ? s : -INFINITY;
      // wave-wide running max over the 8 keys of this step
      float smax = fmaxf(s, __shfl_xor(s, 8, kWave));
      smax = fmaxf(smax, __shfl_xor(smax, 16, kWave));
      smax = fmaxf(smax, __shfl_xor(smax, 32, kWave));
      const float mn = fmaxf(m[j], smax);
      const float corr = exp2f(m[j] - mn);
      const float p = valid ? exp2f(s - mn) : 0.f;
      m[j] = mn;
      l[j] = l[j] * corr + p;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = acc[j][e] * corr + p * vf[e];
    }
  }
  // combine the 8 key groups of the wave (lanes with equal kl), then the waves
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    float lj = l[j];
    lj += __shfl_xor(lj, 8, kWave);
    lj += __shfl_xor(lj, 16, kWave);
    lj += __shfl_xor(lj, 32, kWave);
    l[j] = lj;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float a = acc[j][e];
      a += __shfl_xor(a, 8, kWave);
      a += __shfl_xor(a, 16, kWave);
      a += __shfl_xor(a, 32, kWave);
      acc[j][e] = a;
    }
  }
  if (kr == 0) {
#pragma unroll
    for (int j = 0; j < GROUP; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) S.acc[wave][j][kl * 16 + e] = acc[j][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      S.m[wave][j] = m[j];
      S.l[wave][j] = l[j];
    }
  }
  __syncthreads();
  float *pbase = A.part + ((((size_t)row * A.nkv + g) * kMaxChunks + c) * GROUP) * kPartStride;
  for (int idx = threadIdx.x; idx < GROUP * kHeadDim; idx += 256) {
    const int j = idx / kHeadDim, d = idx % kHeadDim;
    float M = S.m[0][j];
    for (int w = 1; w < 4; ++w) M = fmaxf(M, S.m[w][j]);
    float a = 0.f, ls = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float sc = S.m[w][j] == -INFINITY ? 0.f : exp2f(S.m[w][j] - M);
      a += sc * S.acc[w][j][d];
      ls += sc * S.l[w][j];
    }
    pbase[j * kPartStride + d] = a;
    if (d == 0) {
      pbase[j * kPartStride + 128] = M;
      pbase[j * kPartStride + 129] = ls;
    }
  }

  // the last item of (row, g) to finish merges the chunks in increasing order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  uint32_t *ctr = A.mctr + (size_t)row * A.nkv + g;
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    S.flag = (old == (uint32_t)(nch - 1));
  }
  __syncthreads();
  if (S.flag) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const float *p0 = A.part + (((size_t)row * A.nkv + g) * kMaxChunks * GROUP) * kPartStride;
    const size_t cstride = (size_t)GROUP * kPartStride;
    for (int idx = threadIdx.x; idx < GROUP * nch; idx += 256) {
      const int j = idx / nch, cc = idx % nch;
      S.mc[j][cc] = p0[cc * cstride + j * kPartStride + 128];
      S.lc[j][cc] = p0[cc * cstride + j * kPartStride + 129];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < GROUP * kHeadDim; idx += 256) {
      const int j = idx / kHeadDim, d = idx % kHeadDim;
      float M = -INFINITY;
      for (int cc = 0; cc < nch; ++cc) M = fmaxf(M, S.mc[j][cc]);
      float ls = 0.f, a = 0.f;
      const float *pd = p0 + j * kPartStride + d;
#pragma unroll 8
      for (int cc = 0; cc < nch; ++cc) {
        const float w = exp2f(S.mc[j][cc] - M);
        ls += w * S.lc[j][cc];
        a += w * pd[cc * cstride];
      }
      A.att[((size_t)row * A.nq + g * GROUP + j) * kHeadDim + d] = a / ls;
    }
    if (threadIdx.x == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// ---------------------------------------------------------------- phase D: o_proj
//
// Same structure as phase A with the attention output att[row][nq d] (fp32) as
// input.  Rows that could not be appended (capacity, bad slot) get NaN.
template <int DT, int KV, int RB, int RPW>
__device__ void oproj_tile(const LayerArgs &A, int tile, const uint4 (&wr)[RPW][KV]) {
  const int wave = wave_id(), lane = lane_id();
  const int o0 = (tile * 4 + wave) * RPW;
  const int K = A.nq * kHeadDim;
  for (int rb = 0; rb < A.rows; rb += RB) {
    float x[RB][KV * 8];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = rb + r;
#pragma unroll
      for (int v = 0; v < KV; ++v) {
        if (row < A.rows) {
          const float4 *src = reinterpret_cast<const float4 *>(A.att + (size_t)row * K + (v * 64 + lane) * 8);
          const float4 f0 = src[0], f1 = src[1];
          x[r][v * 8 + 0] = f0.x; x[r][v * 8 + 1] = f0.y; x[r][v * 8 + 2] = f0.z; x[r][v * 8 + 3] = f0.w;
          x[r][v * 8 + 4] = f1.x; x[r][v * 8 + 5] = f1.y; x[r][v * 8 + 6] = f1.z; x[r][v * 8 + 7] = f1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[r][v * 8 + e] = 0.f;
        }
      }
    }
    float acc[RPW][RB];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[i][r] = 0.f;
#pragma unroll
      for (int v = 0; v < KV; ++v) {
        float wf[8];
        unpack8<DT>(wr[i][v], wf);
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][r] += wf[e] * x[r][v * 8 + e];
      }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int r = 0; r < RB; ++r) acc[i][r] = wave_sum(acc[i][r]);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = rb + r;
      if (row < A.rows && lane < RPW) {
        float val = acc[0][r];
#pragma unroll
        for (int i = 1; i < RPW; ++i)
          if (lane == i) val = acc[i][r];
        const size_t o = (size_t)row * A.H + o0 + lane;
        if (A.residual) val += cvt16<DT>(A.residual[o]);
        if (!A.rowtab[row].x) val = __builtin_nanf("");
        if (A.out_f32) reinterpret_cast<float *>(A.out)[o] = val;
        else reinterpret_cast<uint16_t *>(A.out)[o] = rne16<DT>(val);
      }
    }
  }
}

template <int KV, int RPW>
__device__ __forceinline__ void load_wo(const LayerArgs &A, int tile, uint4 (&wr)[RPW][KV]) {
  const int wave = wave_id(), lane = lane_id();
  const int o0 = (tile * 4 + wave) * RPW;
  const int K = A.nq * kHeadDim;
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int v = 0; v < KV; ++v) wr[i][v] = ld16_stream(A.w_o + (size_t)(o0 + i) * K + (v * 64 + lane) * 8);
}

// lengths advance once every earlier phase has read them
__device__ void advance_lengths(const LayerArgs &A) {
  for (int b = threadIdx.x; b < A.B; b += blockDim.x) {
    const int4 rec = A.rowtab[b * A.n];
    if (rec.x) {
      A.lens[rec.z] = rec.y + A.n;
    } else if (A.status) {
      atomicOr(A.status, rec.w ? (uint32_t)ASR_STATUS_CAPACITY : kStatusBadSlot);
    }
  }
}

// ---------------------------------------------------------------- grid barrier (fused dispatch)
//
// bar[0] counts arrivals, bar[1] is a generation number.  The last arriver
// resets the count and bumps the generation; the others wait for the
// generation to move.  Both words return to a reusable state, so the barrier
// needs no reset between calls.  A bounded wait: on timeout the status bit is
// set and the caller stops working (its outputs are then undefined).
__device__ bool grid_barrier(uint32_t *bar, uint32_t nblocks, uint32_t *status, int *s_ok) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = 1;
    const uint32_t gen0 = __hip_atomic_load(&bar[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t old = __hip_atomic_fetch_add(&bar[0], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == nblocks - 1) {
      __hip_atomic_store(&bar[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&bar[1], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const long long start = wall_clock64();
      while (__hip_atomic_load(&bar[1], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen0) {
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - start > kBarrierTimeoutTicks) {
          ok = 0;
          if (status) atomicOr(status, (uint32_t)ASR_STATUS_SYNC_TIMEOUT);
          break;
        }
      }
    }
    *s_ok = ok;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return *s_ok != 0;
}

// ---------------------------------------------------------------- kernels

template <int DT, int KV, int RB, int RPW>
__global__ __launch_bounds__(256) void k_qkv(LayerArgs A) {
  if (blockIdx.x == 0) write_row_table(A);
  qkv_tile<DT, KV, RB, RPW>(A, blockIdx.x);
}

template <int DT, int GROUP>
__global__ __launch_bounds__(256) void k_attn(LayerArgs A) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ AttnShared<GROUP> S;
  uint16_t *knew = reinterpret_cast<uint16_t *>(dyn);
  uint16_t *vnew = knew + A.n * kHeadDim;
  int *pre = reinterpret_cast<int *>(vnew + A.n * kHeadDim);
  build_item_prefix(A, pre, S.wsum);
  const int total = pre[A.rows];
  for (int item = blockIdx.x; item < total; item += gridDim.x) attn_item<DT, GROUP>(A, item, pre, knew, vnew, S);
}

template <int DT, int KV, int RB, int RPW>
__global__ __launch_bounds__(256) void k_oproj(LayerArgs A) {
  if (blockIdx.x == 0) advance_lengths(A);
  uint4 wr[RPW][KV];
  load_wo<KV, RPW>(A, blockIdx.x, wr);
  oproj_tile<DT, KV, RB, RPW>(A, blockIdx.x, wr);
}

// All three phases in one persistent dispatch.  Each block prefetches the
// o_proj weights of its first phase-D tile at the start, so that traffic
// overlaps phases A and C.
template <int DT, int KVI, int RBI, int RPWI, int KVO, int RBO, int RPWO, int GROUP>
__global__ __launch_bounds__(256) void k_fused(LayerArgs A, int tiles_a, int tiles_d) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ AttnShared<GROUP> S;
  __shared__ int s_ok;
  uint16_t *knew = reinterpret_cast<uint16_t *>(dyn);
  uint16_t *vnew = knew + A.n * kHeadDim;
  int *pre = reinterpret_cast<int *>(vnew + A.n * kHeadDim);
  const int G = gridDim.x;

  uint4 wo[RPWO][KVO];
  const int first_d = blockIdx.x;
  if (first_d < tiles_d) load_wo<KVO, RPWO>(A, first_d, wo);

  if (blockIdx.x == 0) write_row_table(A);
  for (int t = blockIdx.x; t < tiles_a; t += G) qkv_tile<DT, KVI, RBI, RPWI>(A, t);
  if (!grid_barrier(A.bar, G, A.status, &s_ok)) return;

  build_item_prefix(A, pre, S.wsum);
  const int total = pre[A.rows];
  for (int item = blockIdx.x; item < total; item += G) attn_item<DT, GROUP>(A, item, pre, knew, vnew, S);
  if (!grid_barrier(A.bar, G, A.status, &s_ok)) return;

  if (blockIdx.x == 0) advance_lengths(A);
  for (int t = blockIdx.x; t < tiles_d; t += G) {
    if (t != first_d) load_wo<KVO, RPWO>(A, t, wo);
    oproj_tile<DT, KVO, RBO, RPWO>(A, t, wo);
  }
}

// ---------------------------------------------------------------- launch

constexpr int rb_for(int kv) { return kv <= 2 ? 4 : (kv <= 4 ? 2 : 1); }
constexpr int kRpwA = 4;   // phase A rows per wave: tiles of 16 QKV rows
constexpr int kRpwD = 1;   // phase D rows per wave: tiles of 4 output rows

size_t attn_dyn_smem(const LayerArgs &a) {
  return (size_t)a.n * kHeadDim * 2 * sizeof(uint16_t) + (size_t)(a.rows + 1) * sizeof(int);
}

template <int DT, int GROUP>
hipError_t multi_attn(const LayerArgs &a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_attn<DT, GROUP>), dim3(grid), dim3(256), attn_dyn_smem(a), s, a);
  return hipGetLastError();
}

template <int DT, int KVI>
hipError_t multi_qkv(const LayerArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((k_qkv<DT, KVI, rb_for(KVI), kRpwA>), dim3(a.nqkv / (4 * kRpwA)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int KVO>
hipError_t multi_oproj(const LayerArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((k_oproj<DT, KVO, rb_for(KVO), kRpwD>), dim3(a.H / (4 * kRpwD)), dim3(256), 0, s, a);
  return hipGetLastError();
}

#define ASR_KV_SWITCH(val, KVNAME, ...)          \
  switch (val) {                                 \
    case 1: { constexpr int KVNAME = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int KVNAME = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int KVNAME = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int KVNAME = 4; __VA_ARGS__; } break; \
    case 5: { constexpr int KVNAME = 5; __VA_ARGS__; } break; \
    case 6: { constexpr int KVNAME = 6; __VA_ARGS__; } break; \
    case 7: { constexpr int KVNAME = 7; __VA_ARGS__; } break; \
    case 8: { constexpr int KVNAME = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;        \
  }

#define ASR_GROUP_SWITCH(val, GNAME, ...)        \
  switch (val) {                                 \
    case 1: { constexpr int GNAME = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int GNAME = 2; __VA_ARGS__; } break; \
    case 4: { constexpr int GNAME = 4; __VA_ARGS__; } break; \
    case 8: { constexpr int GNAME = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;        \
  }

template <int DT>
hipError_t layer_multi(const LayerArgs &a, int attn_grid, hipStream_t s) {
  hipError_t e = hipSuccess;
  ASR_KV_SWITCH(a.H / 512, KVI, e = multi_qkv<DT, KVI>(a, s));
  if (e != hipSuccess) return e;
  ASR_GROUP_SWITCH(a.group, GR, e = multi_attn<DT, GR>(a, attn_grid, s));
  if (e != hipSuccess) return e;
  ASR_KV_SWITCH(a.nq * kHeadDim / 512, KVO, e = multi_oproj<DT, KVO>(a, s));
  return e;
}

// The fused kernel is instantiated for the shapes of the pages' models only
// (hidden 1024 or 2048, 16 q heads, GQA group 2); other shapes use the
// stream-ordered kernels.
bool fused_supported(const LayerArgs &a) {
  return (a.H == 1024 || a.H == 2048) && a.nq == 16 && a.group == 2;
}

template <int DT, int KVI>
hipError_t fused_launch(const LayerArgs &a, int grid, hipStream_t s) {
  constexpr int KVO = 4;  // nq d = 2048
  auto kern = k_fused<DT, KVI, rb_for(KVI), kRpwA, KVO, rb_for(KVO), kRpwD, 2>;
  const int tiles_a = a.nqkv / (4 * kRpwA);
  const int tiles_d = a.H / (4 * kRpwD);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), attn_dyn_smem(a), s, a, tiles_a, tiles_d);
  return hipGetLastError();
}

template <int DT>
hipError_t layer_fused(const LayerArgs &a, int grid, hipStream_t s) {
  if (a.H == 1024) return fused_launch<DT, 2>(a, grid, s);
  return fused_launch<DT, 4>(a, grid, s);
}

}  // namespace

hipError_t launch_layer_multi(const LayerArgs &a, int dtype, int attn_grid, hipStream_t s) {
  return dtype == ASR_BF16 ? layer_multi<ASR_BF16>(a, attn_grid, s) : layer_multi<ASR_F16>(a, attn_grid, s);
}

bool layer_fused_supported(const LayerArgs &a) { return fused_supported(a); }

hipError_t launch_layer_fused(const LayerArgs &a, int dtype, int grid, hipStream_t s) {
  return dtype == ASR_BF16 ? layer_fused<ASR_BF16>(a, grid, s) : layer_fused<ASR_F16>(a, grid, s);
}

// Largest grid of the fused kernel that is co-resident on the device: blocks
// per CU from the occupancy calculator times the CU count.
int fused_max_grid(int dtype, int H, size_t dyn_smem, int cus) {
  int per_cu = 0;
  hipError_t e;
  if (dtype == ASR_BF16) {
    e = H == 1024 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &per_cu, k_fused<ASR_BF16, 2, 4, kRpwA, 4, 2, kRpwD, 2>, 256, dyn_smem)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &per_cu, k_fused<ASR_BF16, 4, 2, kRpwA, 4, 2, kRpwD, 2>, 256, dyn_smem);
  } else {
    e = H == 1024 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &per_cu, k_fused<ASR_F16, 2, 4, kRpwA, 4, 2, kRpwD, 2>, 256, dyn_smem)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &per_cu, k_fused<ASR_F16, 4, 2, kRpwA, 4, 2, kRpwD, 2>, 256, dyn_smem);
  }
  if (e != hipSuccess || per_cu <= 0) return 0;
  return per_cu * cus;
}

size_t layer_dyn_smem(const LayerArgs &a) { return attn_dyn_smem(a); }

}  // namespace asr
