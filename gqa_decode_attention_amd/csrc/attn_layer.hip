// Phase kernels of one attention-block layer call (decode or k-token verify).
//
// Phases, in stream order:
//   1. k_qkv    input RMSNorm fused into the q/k/v projection (GEMV over rows)
//   2. k_prep   per-head RMSNorm of q and k, rotary, rounding of k/v into the cache
//   3. k_attn   split-KV attention: one workgroup per (row, kv head, chunk of keys),
//               both q heads of the kv head share each K/V row; partial (m, l, acc)
//   4. k_merge  log-sum-exp merge of the chunk partials in a fixed order
//   5. k_oproj  output projection (+ residual); lengths advanced
//
// The operation list follows "Qwen3-ASR -- Latency & Bottleneck Analysis",
// section 07 (q/k/v projections, GQA repeat_kv, QK^T, fp32 softmax, AV, o_proj)
// and its norm and rotary rows; the causal rule of verify rows follows "Can CTC
// make Qwen3-ASR faster?", section 03 (position i sees the committed prefix and
// the candidates before it, and itself).
#include "device_common.h"
#include "internal.h"

namespace asr {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

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

// ---------------------------------------------------------------- phase 1: QKV projection
//
// Wave w of block b owns RPW consecutive output rows; their weights stay in
// registers while the wave walks over the input rows RB at a time.  Lane l
// covers columns (v * 64 + l) * 8 .. + 7 for v < KV, so every wave-wide load
// reads 1 KB contiguously.  RMSNorm: h = x * g * rsqrt(mean(x^2) + eps).
template <int DT, int KV, int RB, int RPW>
__global__ __launch_bounds__(256) void k_qkv(LayerArgs A) {
  const int wave = wave_id(), lane = lane_id();
  const int o0 = (blockIdx.x * 4 + wave) * RPW;
  if (o0 >= A.nqkv) return;
  const int H = A.H;
  float g[KV * 8];
#pragma unroll
  for (int v = 0; v < KV; ++v) unpack8<DT>(ld16(A.g_in + (v * 64 + lane) * 8), g + v * 8);
  uint4 wr[RPW][KV];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int v = 0; v < KV; ++v)
      wr[i][v] = ld16_stream(A.w_qkv + (size_t)(o0 + i) * H + (v * 64 + lane) * 8);

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

// ---------------------------------------------------------------- phase 2: head prep
//
// One wave per (row, head).  Lane t holds the rotary pair (t, t + 64).
// q heads: RMSNorm * g_q, rotate, scale by log2(e)/sqrt(d) (scores then live in
// the log2 domain), store fp32.  k heads: RMSNorm * g_k, rotate, round into the
// cache at position L + r.  v heads: round into the cache.
template <int DT>
__global__ __launch_bounds__(256) void k_prep(LayerArgs A) {
  const int wave = wave_id(), lane = lane_id();
  const int row = blockIdx.x;
  const int head = blockIdx.y * 4 + wave;
  const RowInfo ri = row_info(A, row);
  if (blockIdx.y == 0 && threadIdx.x == 0 && !ri.ok && A.status)
    atomicOr(A.status, ri.slot_ok ? (uint32_t)ASR_STATUS_CAPACITY : kStatusBadSlot);
  if (head >= A.nq + 2 * A.nkv) return;
  const float *src = A.qkv + (size_t)row * A.nqkv + head * kHeadDim;
  float u0 = src[lane], u1 = src[lane + 64];
  if (head < A.nq + A.nkv) {
    const float ss = wave_sum(u0 * u0 + u1 * u1);
    const float inv = 1.0f / sqrtf(ss / (float)kHeadDim + A.eps);
    const uint16_t *gp = head < A.nq ? A.g_q : A.g_k;
    u0 *= cvt16<DT>(gp[lane]) * inv;
    u1 *= cvt16<DT>(gp[lane + 64]) * inv;
    // angle = pos * theta^(-2 lane / d), formed in fp64, then rotated in fp32
    const double omega = exp2(-(2.0 * lane / kHeadDim) * log2((double)A.theta));
    double sn, cs;
    sincos((double)ri.pos * omega, &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const float r0 = u0 * c - u1 * s;
    const float r1 = u1 * c + u0 * s;
    if (head < A.nq) {
      const float qs = kLog2e * rsqrtf((float)kHeadDim);
      float *dst = A.qn + ((size_t)row * A.nq + head) * kHeadDim;
      dst[lane] = r0 * qs;
      dst[lane + 64] = r1 * qs;
    } else if (ri.ok) {
      const int g = head - A.nq;
      uint16_t *dst = A.kc + (((size_t)ri.slot * A.nkv + g) * A.capacity + ri.L + ri.r) * kHeadDim;
      dst[lane] = rne16<DT>(r0);
      dst[lane + 64] = rne16<DT>(r1);
    }
  } else if (ri.ok) {
    const int g = head - A.nq - A.nkv;
    uint16_t *dst = A.vc + (((size_t)ri.slot * A.nkv + g) * A.capacity + ri.L + ri.r) * kHeadDim;
    dst[lane] = rne16<DT>(u0);
    dst[lane + 64] = rne16<DT>(u1);
  }
}

// ---------------------------------------------------------------- phase 3: split-KV attention
//
// Work items are (row, kv head g, chunk c) for every chunk of `split` keys that
// holds a visible key; a block-wide prefix sum over the rows' chunk counts
// (computed on the device from lens, so no host readback) turns a flat item id
// into its (row, g, c).  Blocks stride over the items.
//
// Inside an item: lanes form groups of 8; a group owns one key row (8 lanes x
// 16 dims = 128 dims, 256 contiguous bytes), a wave covers 8 rows, the block
// 32.  Pass 1 computes the GROUP scores of every key (all q heads of the kv
// head reuse the loaded row) into LDS; then per head m = max, p = exp2(s - m),
// l = sum p; pass 2 accumulates p * V the same way.  The partial (acc, m, l)
// of each q head goes to the workspace.
__device__ __forceinline__ int chunks_of(int nvis, int split) { return (nvis + split - 1) / split; }

template <int DT, int GROUP>
__global__ __launch_bounds__(256) void k_attn(LayerArgs A) {
  extern __shared__ int s_pre[];                 // [rows + 1] item prefix
  __shared__ float s_sc[GROUP][kMaxSplit];       // scores, then probabilities
  __shared__ float s_acc[4][GROUP][kHeadDim];
  __shared__ float s_ml[GROUP][2];
  __shared__ int s_wsum[4];
  const int wave = wave_id(), lane = lane_id();
  const int rows = A.rows;

  // prefix over rows of (chunks per row) * nkv
  {
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
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    int run = base + incl - local;
    for (int i = beg; i < end; ++i) {
      s_pre[i] = run;
      run += chunks_of(row_info(A, i).nvis, A.split) * A.nkv;
    }
    if (threadIdx.x == 255) s_pre[rows] = run;
    __syncthreads();
  }
  const int total = s_pre[rows];
  const int kl = lane & 7, kr = lane >> 3;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = rows;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] <= item) lo = mid; else hi = mid;
    }
    const int row = lo;
    const int nch = (s_pre[row + 1] - s_pre[row]) / A.nkv;
    const int rem = item - s_pre[row];
    const int g = rem / nch, c = rem - g * nch;
    const RowInfo ri = row_info(A, row);
    const int t0 = c * A.split, t1 = min(t0 + A.split, ri.nvis);

    float q[GROUP][16];
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      const float4 *qp = reinterpret_cast<const float4 *>(
          A.qn + ((size_t)row * A.nq + g * GROUP + j) * kHeadDim + kl * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 f = qp[e];
        q[j][4 * e] = f.x; q[j][4 * e + 1] = f.y; q[j][4 * e + 2] = f.z; q[j][4 * e + 3] = f.w;
      }
    }
    const size_t kvrow0 = ((size_t)ri.slot * A.nkv + g) * A.capacity;
    const uint16_t *Kp = A.kc + kvrow0 * kHeadDim + kl * 16;
    const uint16_t *Vp = A.vc + kvrow0 * kHeadDim + kl * 16;

    // pass 1: scores
    for (int tb = t0 + wave * 8; tb < t1; tb += 32) {
      const int t = tb + kr;
      const bool valid = t < t1;
      const int tc = valid ? t : t1 - 1;
      float kf[16];
      unpack8<DT>(ld16_stream(Kp + (size_t)tc * kHeadDim), kf);
      unpack8<DT>(ld16_stream(Kp + (size_t)tc * kHeadDim + 8), kf + 8);
#pragma unroll
      for (int j = 0; j < GROUP; ++j) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) s += q[j][e] * kf[e];
        s = group_sum<8>(s);
        if (valid && kl == 0) s_sc[j][t - t0] = s;
      }
    }
    __syncthreads();
    const int nk = t1 - t0;
    for (int j = wave; j < GROUP; j += 4) {
      float m = -INFINITY;
      for (int i = lane; i < nk; i += kWave) m = fmaxf(m, s_sc[j][i]);
      m = wave_max(m);
      float l = 0.f;
      for (int i = lane; i < nk; i += kWave) {
        const float p = exp2f(s_sc[j][i] - m);
        s_sc[j][i] = p;
        l += p;
      }
      l = wave_sum(l);
      if (lane == 0) { s_ml[j][0] = m; s_ml[j][1] = l; }
    }
    __syncthreads();

    // pass 2: p * V
    float acc[GROUP][16];
#pragma unroll
    for (int j = 0; j < GROUP; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    for (int tb = t0 + wave * 8; tb < t1; tb += 32) {
      const int t = tb + kr;
      const bool valid = t < t1;
      const int tc = valid ? t : t1 - 1;
      float vf[16];
      unpack8<DT>(ld16_stream(Vp + (size_t)tc * kHeadDim), vf);
      unpack8<DT>(ld16_stream(Vp + (size_t)tc * kHeadDim + 8), vf + 8);
#pragma unroll
      for (int j = 0; j < GROUP; ++j) {
        const float p = valid ? s_sc[j][tc - t0] : 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] += p * vf[e];
      }
    }
#pragma unroll
    for (int j = 0; j < GROUP; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float a = acc[j][e];
        a += __shfl_xor(a, 8, kWave);
        a += __shfl_xor(a, 16, kWave);
        a += __shfl_xor(a, 32, kWave);
        acc[j][e] = a;
      }
    if (kr == 0) {
#pragma unroll
      for (int j = 0; j < GROUP; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s_acc[wave][j][kl * 16 + e] = acc[j][e];
    }
    __syncthreads();
    float *pbase = A.part + ((((size_t)row * A.nkv + g) * kMaxChunks + c) * GROUP) * kPartStride;
    for (int idx = threadIdx.x; idx < GROUP * kHeadDim; idx += 256) {
      const int j = idx / kHeadDim, d = idx % kHeadDim;
      pbase[j * kPartStride + d] = s_acc[0][j][d] + s_acc[1][j][d] + s_acc[2][j][d] + s_acc[3][j][d];
    }
    if (threadIdx.x < GROUP) {
      pbase[threadIdx.x * kPartStride + 128] = s_ml[threadIdx.x][0];
      pbase[threadIdx.x * kPartStride + 129] = s_ml[threadIdx.x][1];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- phase 4: merge
//
// a = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c with M = max_c m_c, over
// the chunks in increasing order (deterministic).  Rows that could not be
// appended get NaN.
template <int GROUP>
__global__ __launch_bounds__(128) void k_merge(LayerArgs A) {
  const int row = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const RowInfo ri = row_info(A, row);
  float *dst = A.att + ((size_t)row * A.nq + h) * kHeadDim + d;
  if (!ri.ok) {
    *dst = __builtin_nanf("");
    return;
  }
  const int nch = chunks_of(ri.nvis, A.split);
  const int g = h / GROUP, j = h % GROUP;
  const float *p = A.part + (((size_t)row * A.nkv + g) * kMaxChunks * GROUP + j) * kPartStride;
  const size_t cstride = (size_t)GROUP * kPartStride;
  float M = -INFINITY;
  for (int c = 0; c < nch; ++c) M = fmaxf(M, p[c * cstride + 128]);
  float l = 0.f, a = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float w = exp2f(p[c * cstride + 128] - M);
    l += w * p[c * cstride + 129];
    a += w * p[c * cstride + d];
  }
  *dst = a / l;
}

// ---------------------------------------------------------------- phase 5: o_proj
//
// Same structure as phase 1 with input att[row][nq d] (fp32).  Block 0 also
// advances lens[slot] by n for every sequence that was appended; nothing else
// in this kernel reads lens, and every earlier phase has finished reading it.
template <int DT, int KV, int RB, int RPW>
__global__ __launch_bounds__(256) void k_oproj(LayerArgs A) {
  if (blockIdx.x == 0) {
    for (int b = threadIdx.x; b < A.B; b += 256) {
      const RowInfo ri = row_info(A, b * A.n);
      if (ri.ok) A.lens[ri.slot] = ri.L + A.n;
    }
  }
  const int wave = wave_id(), lane = lane_id();
  const int o0 = (blockIdx.x * 4 + wave) * RPW;
  if (o0 >= A.H) return;
  const int K = A.nq * kHeadDim;
  uint4 wr[RPW][KV];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int v = 0; v < KV; ++v) wr[i][v] = ld16_stream(A.w_o + (size_t)(o0 + i) * K + (v * 64 + lane) * 8);

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
        if (A.out_f32) reinterpret_cast<float *>(A.out)[o] = val;
        else reinterpret_cast<uint16_t *>(A.out)[o] = rne16<DT>(val);
      }
    }
  }
}

// ---------------------------------------------------------------- launch

template <int DT, int KV>
hipError_t launch_proj_in(const LayerArgs &a, hipStream_t s) {
  constexpr int RB = KV <= 2 ? 4 : (KV <= 4 ? 2 : 1);
  constexpr int RPW = 4;
  hipLaunchKernelGGL((k_qkv<DT, KV, RB, RPW>), dim3(a.nqkv / (4 * RPW)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT, int KV>
hipError_t launch_proj_out(const LayerArgs &a, hipStream_t s) {
  constexpr int RB = KV <= 2 ? 4 : (KV <= 4 ? 2 : 1);
  constexpr int RPW = 4;
  hipLaunchKernelGGL((k_oproj<DT, KV, RB, RPW>), dim3(a.H / (4 * RPW)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t proj_in(const LayerArgs &a, hipStream_t s) {
  switch (a.H / 512) {
    case 1: return launch_proj_in<DT, 1>(a, s);
    case 2: return launch_proj_in<DT, 2>(a, s);
    case 3: return launch_proj_in<DT, 3>(a, s);
    case 4: return launch_proj_in<DT, 4>(a, s);
    case 5: return launch_proj_in<DT, 5>(a, s);
    case 6: return launch_proj_in<DT, 6>(a, s);
    case 7: return launch_proj_in<DT, 7>(a, s);
    case 8: return launch_proj_in<DT, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t proj_out(const LayerArgs &a, hipStream_t s) {
  switch (a.nq * kHeadDim / 512) {
    case 1: return launch_proj_out<DT, 1>(a, s);
    case 2: return launch_proj_out<DT, 2>(a, s);
    case 3: return launch_proj_out<DT, 3>(a, s);
    case 4: return launch_proj_out<DT, 4>(a, s);
    case 5: return launch_proj_out<DT, 5>(a, s);
    case 6: return launch_proj_out<DT, 6>(a, s);
    case 7: return launch_proj_out<DT, 7>(a, s);
    case 8: return launch_proj_out<DT, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int DT, int GROUP>
hipError_t attn_and_merge(const LayerArgs &a, int attn_grid, hipStream_t s) {
  const size_t shmem = (size_t)(a.rows + 1) * sizeof(int);
  hipLaunchKernelGGL((k_attn<DT, GROUP>), dim3(attn_grid), dim3(256), shmem, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_merge<GROUP>), dim3(a.rows, a.nq), dim3(128), 0, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t layer_multi(const LayerArgs &a, int attn_grid, hipStream_t s) {
  hipError_t e = proj_in<DT>(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_prep<DT>), dim3(a.rows, (a.nq + 2 * a.nkv + 3) / 4), dim3(256), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (a.group) {
    case 1: e = attn_and_merge<DT, 1>(a, attn_grid, s); break;
    case 2: e = attn_and_merge<DT, 2>(a, attn_grid, s); break;
    case 4: e = attn_and_merge<DT, 4>(a, attn_grid, s); break;
    case 8: e = attn_and_merge<DT, 8>(a, attn_grid, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return proj_out<DT>(a, s);
}

}  // namespace

hipError_t launch_layer_multi(const LayerArgs &a, int dtype, int attn_grid, hipStream_t s) {
  return dtype == ASR_BF16 ? layer_multi<ASR_BF16>(a, attn_grid, s) : layer_multi<ASR_F16>(a, attn_grid, s);
}

}  // namespace asr
