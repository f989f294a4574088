// One attention-block layer call (decode or k-token verify) on gfx950.
//
// Phases; each is a loop over independent work items, written as device
// functions shared by both dispatch modes:
//   A. QKV tiles   input RMSNorm fused into the q/k/v projection.  A tile is 16
//                  output rows = 8 rotary pairs (t, t + 64) of one head, for all
//                  input rows: it applies the q/k norm gain and the rotary to its
//                  pairs and stores the partial sum of squares of its raw rows;
//                  v rows are stored raw.  Above 4 rows the projection runs on
//                  MFMA (k_qkv_mfma) with the same tile and epilogue.
//   C. attention   one item per (row, kv head g, chunk of keys): all q heads of g
//                  share every K/V row of the chunk; the q/k norms are finished
//                  with the tiles' partial sums; the rows this call appends are
//                  rounded once, taken from LDS and written to the cache by the
//                  item of the sequence's last row; single-pass online softmax;
//                  a partial (m, l, acc) per q head.  The last item of a (row, g)
//                  to finish merges the chunks (log-sum-exp, fixed order) into
//                  the attention output.
//   D. o_proj      output projection (+ residual); lengths advanced.
// ASR_DISPATCH_MULTI runs the phases as kernels in stream order; a kernel
// boundary makes each phase's results visible to the next.
// ASR_DISPATCH_FUSED runs them in one persistent kernel (k_flow) whose resident
// workgroups order the phases through counters in the workspace; data crossing
// workgroups inside it go through device-coherent accesses (st_dev / ld_dev,
// ld_dev4).
//
// The operation list follows "Qwen3-ASR -- Latency & Bottleneck Analysis",
// section 07 (q/k/v projections, GQA repeat_kv, QK^T, fp32 softmax, AV, o_proj)
// with the norms of "Norms are real money at this size" and the fp32 rotary of
// the section 03 table.  The causal rule of verify rows follows "Can CTC make
// Qwen3-ASR faster?", section 03: position i sees the committed prefix and the
// candidates up to i.
#include <hip/hip_ext.h>

#include <atomic>

#include "device_common.h"
#include "internal.h"

namespace asr {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr long long kBarrierTimeoutTicks = 50000000;   // wall clock ticks: 0.5 s at the 100 MHz constant clock
                                                      // gfx9 parts report (hipDeviceAttributeWallClockRate)
constexpr int kRpwA = 4;                              // phase A rows per wave: tiles of 16 rows
constexpr int kTilesPerHead = kHeadDim / (4 * kRpwA); // 8
constexpr int kRpwD = 1;                              // phase D rows per wave: tiles of 4 rows

// ---------------------------------------------------------------- coherence-selected accesses
template <bool COH> __device__ __forceinline__ float ldx(const float *p) {
  if constexpr (COH) return ld_dev(p); else return *p;
}
template <bool COH> __device__ __forceinline__ void stx(float *p, float v) {
  if constexpr (COH) st_dev(p, v); else *p = v;
}
template <bool COH> __device__ __forceinline__ void stx16(uint16_t *p, uint16_t v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); else *p = v;
}
template <bool COH> __device__ __forceinline__ uint4 ldx16B(const uint16_t *p) {
  if constexpr (COH) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
    return make_uint4(ld_dev(q), ld_dev(q + 1), ld_dev(q + 2), ld_dev(q + 3));
  } else {
    return ld16_stream(p);
  }
}

// Rows of a call, sequence-major: sequence b owns rows [seq_row0(b), seq_row0(b) + seq_rows(b)),
// n each, or (MIX: kernels of a mixed call) the host's block sizes.  MIX is a template argument
// so that the kernels of uniform calls carry no trace of the mixed layout.
template <bool MIX = false>
__device__ __forceinline__ int seq_row0(const LayerArgs &A, int b) {
  if constexpr (MIX) return A.qo[b];
  else return b * A.n;
}
template <bool MIX = false>
__device__ __forceinline__ int seq_rows(const LayerArgs &A, int b) {
  if constexpr (MIX) return A.qo[b + 1] - A.qo[b];
  else return A.n;
}

// sequence of row `row`: a division, or in a mixed call the last b with qo[b] <= row
// (a binary search over at most kVmMaxSeqs starts)
template <bool MIX = false>
__device__ __forceinline__ int seq_of(const LayerArgs &A, int row) {
  if constexpr (!MIX) {
    return row / A.n;
  } else {
    int b = 0;
#pragma unroll
    for (int step = kVmMaxSeqs / 2; step > 0; step >>= 1)
      if (b + step < A.B && A.qo[b + step] <= row) b += step;
    return b;
  }
}

struct RowInfo {
  int b, slot, L, pos, nvis, r;
  bool ok, slot_ok;
};

// Row `row` = (sequence b, block offset r).  Visible keys: L + r + 1.
template <bool MIX = false>
__device__ __forceinline__ RowInfo row_info(const LayerArgs &A, int row) {
  RowInfo ri;
  const int b = seq_of<MIX>(A, row);
  ri.b = b;
  ri.r = row - seq_row0<MIX>(A, b);
  const int s = A.slots ? A.slots[b] : b;
  ri.slot = s;
  ri.slot_ok = (s >= 0 && s < A.batch_cap);
  const int L = ri.slot_ok ? A.lens[s] : 0;
  ri.L = L;
  ri.ok = ri.slot_ok && L >= 0 && L + seq_rows<MIX>(A, b) <= A.capacity;
  ri.pos = (A.positions ? A.positions[b] : L) + ri.r;
  ri.nvis = ri.ok ? L + ri.r + 1 : 0;
  return ri;
}

__device__ __forceinline__ int chunks_of(int nvis, int split) { return (nvis + split - 1) / split; }

// Rotary position of pair t of row `row`: the row's position, or with
// multi-section rotary the position component of t's section (positions
// [3][B]; NULL: the length), plus the row's offset in its block.
template <bool MIX = false>
__device__ __forceinline__ int rope_pos(const LayerArgs &A, int row, int t) {
  const RowInfo ri = row_info<MIX>(A, row);
  if (!A.mrope) return ri.pos;
  const int c = t < A.ms0 ? 0 : (t < A.ms0 + A.ms1 ? 1 : 2);
  return (A.positions ? A.positions[c * A.B + ri.b] : ri.L) + ri.r;
}

// Row table for phases M and D (which must not read lens: lengths change in D).
template <bool COH, bool MIX = false>
__device__ void write_row_table(const LayerArgs &A) {
  for (int row = threadIdx.x; row < A.rows; row += blockDim.x) {
    const RowInfo ri = row_info<MIX>(A, row);
    int *rec = reinterpret_cast<int *>(A.rowtab + row);
    if constexpr (COH) {
      st_dev(rec + 0, (int)ri.ok);
      st_dev(rec + 1, ri.L);
      st_dev(rec + 2, ri.slot);
      st_dev(rec + 3, (int)ri.slot_ok);
    } else {
      A.rowtab[row] = make_int4(ri.ok, ri.L, ri.slot, ri.slot_ok);
    }
  }
}

template <bool COH>
__device__ __forceinline__ int4 read_row_table(const LayerArgs &A, int row) {
  if constexpr (COH) {
    const int *rec = reinterpret_cast<const int *>(A.rowtab + row);
    return make_int4(ld_dev(rec), ld_dev(rec + 1), ld_dev(rec + 2), ld_dev(rec + 3));
  } else {
    return A.rowtab[row];
  }
}

// ---------------------------------------------------------------- phase A: QKV projection
//
// RMSNorm of q and k is a per-head scalar, so rotary can act before it:
// rotate(g * q / rms) = rotate(g * q) / rms.  A tile therefore owns whole rotary
// pairs: tile j of head h holds pair indices t in [8 jj, 8 jj + 8) (jj = j % 8),
// i.e. the output rows h*128 + t and h*128 + 64 + t; wave w takes two pairs.
// For q and k heads the tile stores u = rotate(gain * qk_raw) and the partial sum
// of squares of its raw rows; the consumer finishes with u / sqrt(sum/d + eps).
// v heads are stored raw.  Rotary: pair t at position pos turns by
// pos * theta^(-2t/d); the angle and its cosine and sine are formed in fp64.
//
// Lane l covers input columns (v * 64 + l) * 8 .. + 7 for v < KV, so every
// wave-wide load reads 1 KB contiguously; the wave's four weight rows stay in
// registers while it walks over the input rows RB at a time.
// Input RMSNorm: h = x * g_in / sqrt(mean(x^2) + eps).
__device__ __forceinline__ void qkv_tile_rows(int tile, int (&orow)[4]) {
  const int head = tile / kTilesPerHead, jj = tile % kTilesPerHead;
  const int ta = 8 * jj + 2 * wave_id(), tb = ta + 1;
  orow[0] = head * kHeadDim + ta;
  orow[1] = head * kHeadDim + ta + 64;
  orow[2] = head * kHeadDim + tb;
  orow[3] = head * kHeadDim + tb + 64;
}

// the wave's four weight rows of tile `tile`
template <int KV>
__device__ __forceinline__ void qkv_tile_weights(const LayerArgs &A, int tile, uint4 (&wr)[4][KV]) {
  int orow[4];
  qkv_tile_rows(tile, orow);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < KV; ++v)
      wr[i][v] = ld16_stream(A.w_qkv + (size_t)orow[i] * A.H + (v * 64 + lane_id()) * 8);
}

// fp64 rotary angle of pair t at position pos, as (cos, sin)
__device__ __forceinline__ float2 rope_cs(int pos, double omega) {
  double sn, cs;
  sincos((double)pos * omega, &sn, &cs);
  return make_float2((float)cs, (float)sn);
}

// LOADW: the tile requests its weight rows itself and, right behind them and
// before any wait, its small inputs (x of the first RB rows, the input-norm
// gain, the q/k gains), so that all of them travel together (a wait on a load
// waits on every load issued before it: a small load issued only after a
// first wait would add a round trip).  Else the caller has requested the
// weights into wr.
template <int DT, int KV, int RB, bool COH, bool LOADW = false>
__device__ __forceinline__ void qkv_tile(const LayerArgs &A, int tile, float (*s_ssq)[4], uint4 (&wr)[4][KV]) {
  const int wave = wave_id(), lane = lane_id();
  const int head = tile / kTilesPerHead, jj = tile % kTilesPerHead;
  const int ta = 8 * jj + 2 * wave, tb = ta + 1;
  int orow[4];
  qkv_tile_rows(tile, orow);
  const bool rot = head < A.nq + A.nkv;
  const int H = A.H;
  const uint16_t *gp = head < A.nq ? A.g_q : A.g_k;   // v heads: unused
  if constexpr (LOADW) qkv_tile_weights<KV>(A, tile, wr);
  uint4 x0[RB][KV], g16[KV];
  uint32_t gq16[4];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int v = 0; v < KV; ++v) x0[r][v] = ld16(A.x + (size_t)min(r, A.rows - 1) * H + (v * 64 + lane) * 8);
#pragma unroll
  for (int v = 0; v < KV; ++v) g16[v] = ld16(A.g_in + (v * 64 + lane) * 8);
  gq16[0] = gp[ta];
  gq16[1] = gp[ta + 64];
  gq16[2] = gp[tb];
  gq16[3] = gp[tb + 64];
  // rotary angles of the first row block while the loads travel: the rows'
  // positions come through scalar loads, which do not wait on vector loads.
  // Lane 2r computes pair ta of row rb + r, lane 2r + 1 pair tb: each lane
  // selects its position among the block's and takes one fp64 sincos.
  const int tl = (lane & 1) ? tb : ta;
  const double om = exp2(-(2.0 * tl / kHeadDim) * log2((double)A.theta));
  auto angles = [&](int rb, float &cs_c, float &cs_s) __attribute__((always_inline)) {
    cs_c = 1.f;
    cs_s = 0.f;
    if (rot) {
      int pos = 0;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (rb + r < A.rows) {
          const int pa = rope_pos(A, rb + r, ta), pb = rope_pos(A, rb + r, tb);
          if (lane >> 1 == r) pos = (lane & 1) ? pb : pa;
        }
      }
      if ((lane >> 1) < RB && rb + (lane >> 1) < A.rows) {
        const float2 c = rope_cs(pos, om);
        cs_c = c.x;
        cs_s = c.y;
      }
    }
  };
  float cs_c0, cs_s0;
  angles(0, cs_c0, cs_s0);
  __builtin_amdgcn_sched_barrier(0);   // loads and angles before the first use of a loaded value
  float g[KV * 8];
#pragma unroll
  for (int v = 0; v < KV; ++v) unpack8<DT>(g16[v], g + v * 8);
  float gq[4] = {1.f, 1.f, 1.f, 1.f};
  if (rot) {
#pragma unroll
    for (int i = 0; i < 4; ++i) gq[i] = cvt16<DT>((uint16_t)gq16[i]);
  }

  for (int rb = 0; rb < A.rows; rb += RB) {
    float cs_c = cs_c0, cs_s = cs_s0;
    if (rb > 0) angles(rb, cs_c, cs_s);
    float x[RB][KV * 8];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = rb + r;
      float ss = 0.f;
      if (row < A.rows) {
#pragma unroll
        for (int v = 0; v < KV; ++v)
          unpack8<DT>(rb == 0 ? x0[r][v] : ld16(A.x + (size_t)row * H + (v * 64 + lane) * 8), x[r] + v * 8);
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
    float acc[4][RB];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
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
    // Sums over the wave: reduce-scatter over lane bits 5 and 4 (the 16-lane row
    // q = lane >> 4 keeps output row q of the wave), then a sum over the 16 lanes.
    constexpr int N = 4 * RB;
    float v1[N], v2[N / 2], v3[N / 4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < RB; ++r) v1[i * RB + r] = acc[i][r];
    rs_half<N, 32>(v1, v2);
    rs_half<N / 2, 16>(v2, v3);
    const int q = lane >> 4;   // output row orow[q]: rotary pair a (rows 0, 1) or b (rows 2, 3)
    const float gqq = q == 0 ? gq[0] : q == 1 ? gq[1] : q == 2 ? gq[2] : gq[3];
    const int oq = q == 0 ? orow[0] : q == 1 ? orow[1] : q == 2 ? orow[2] : orow[3];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int row = rb + r;
      if (row >= A.rows) continue;
      float o = sum16(v3[r]);
      if (rot) {
        const float ca = readlane(cs_c, 2 * r), sa = readlane(cs_s, 2 * r);
        const float cb = readlane(cs_c, 2 * r + 1), sb = readlane(cs_s, 2 * r + 1);
        const float c = (q >> 1) ? cb : ca, sn = (q >> 1) ? sb : sa;
        float ssq = o * o;
        ssq = xsum<16>(ssq);
        ssq = xsum<32>(ssq);
        const float u = gqq * o;
        const float up = xpart<16>(u);   // the other row of the pair
        o = (q & 1) ? u * c + up * sn : u * c - up * sn;
        if (lane == 0) s_ssq[r][wave] = ssq;
      }
      if ((lane & 15) == 0) stx<COH>(A.qkv + (size_t)row * A.nqkv + oq, o);
    }
    if (rot) {
      __syncthreads();
      if (threadIdx.x < RB && rb + (int)threadIdx.x < A.rows) {
        const int r = threadIdx.x;
        stx<COH>(A.ssq + ((size_t)(rb + r) * (A.nq + A.nkv) + head) * kTilesPerHead + jj,
                 s_ssq[r][0] + s_ssq[r][1] + s_ssq[r][2] + s_ssq[r][3]);
      }
      __syncthreads();
    }
  }
}

// 1 / sqrt(mean of squares + eps) of head `head` of row `row` from the tile partials
// same, from the two 16-byte halves of the 8 partials
__device__ __forceinline__ float inv_rms_of(const LayerArgs &A, float4 a, float4 b) {
  const float s = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
  return 1.0f / sqrtf(s / (float)kHeadDim + A.eps);
}

template <bool COH>
__device__ __forceinline__ float head_inv_rms(const LayerArgs &A, int row, int head) {
  const float *p = A.ssq + ((size_t)row * (A.nq + A.nkv) + head) * kTilesPerHead;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kTilesPerHead; ++j) s += ldx<COH>(p + j);
  return 1.0f / sqrtf(s / (float)kHeadDim + A.eps);
}

// ---------------------------------------------------------------- phase C: attention
//
// Items are (row, kv head g, chunk c) for every chunk of `split` keys that holds
// a visible key of the row.  A block-wide prefix sum over the rows' chunk counts
// (from lens, on the device: no host readback) maps a flat item id to (row, g, c).
//
// Lane layout: groups of 8 lanes; a group owns one key row (8 lanes x 16 dims =
// 128 dims, 256 contiguous bytes); a wave takes 8 keys per step, the block 32.
// Each wave keeps a running max and sum per q head (online softmax), so K and
// V stream once; the 4 waves are combined in LDS at the end of the item.
template <int GROUP>
struct AttnShared {
  float acc[4][GROUP][kHeadDim];
  float m[4][GROUP], l[4][GROUP];
  int wsum[4];
  int flag;
};

// block-wide exclusive prefix of (chunks per row) * nkv (KEYS: visible keys per
// row * nkv) into pre[0..rows]; each row's (slot, committed length, visible
// keys, block offset) is kept in rinfo[] so that work starts without global loads
template <bool KEYS = false, bool MIX = false>
__device__ void build_item_prefix(const LayerArgs &A, int *pre, int4 *rinfo, int *wsum) {
  const int wave = wave_id(), lane = lane_id();
  const int rows = A.rows;
  const int per = (rows + 255) / 256;
  const int beg = min((int)threadIdx.x * per, rows), end = min(beg + per, rows);
  int local = 0;
  for (int i = beg; i < end; ++i) {
    const RowInfo ri = row_info<MIX>(A, i);
    rinfo[i] = make_int4(ri.slot, ri.L, ri.nvis, ri.r);
    local += (KEYS ? ri.nvis : chunks_of(ri.nvis, A.split)) * A.nkv;
  }
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
    run += (KEYS ? rinfo[i].z : chunks_of(rinfo[i].z, A.split)) * A.nkv;
  }
  if (threadIdx.x == 255) pre[rows] = run;
  __syncthreads();
}

struct Item {
  int row, g, c, nch;
};

__device__ __forceinline__ Item decode_item(const LayerArgs &A, int item, const int *pre) {
  int lo = 0, hi = A.rows;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= item) lo = mid; else hi = mid;
  }
  // (an item is uniform over its workgroup: readfirstlane keeps its indices, and the
  // buffer resources built from them, in scalar registers)
  Item it;
  it.row = __builtin_amdgcn_readfirstlane(lo);
  it.nch = __builtin_amdgcn_readfirstlane((pre[lo + 1] - pre[lo]) / A.nkv);
  const int rem = item - __builtin_amdgcn_readfirstlane(pre[lo]);
  it.g = rem / it.nch;
  it.c = rem - it.g * it.nch;
  return it;
}

// Buffer resource for raw 16-byte loads from `base` (bounds: `bytes`).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// the same with the nontemporal hint: a stream read once, kept out of the caches' way
constexpr int kCachePolicyStream = 2;   // nt

__device__ __forceinline__ uint4 ld_buf_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicyStream));
}

// 16 bytes from LDS through an LDS-typed pointer
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_ld16(const uint16_t *p) {
  const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 2^x for the softmax weights (x <= 0 or -inf): the hardware exponential;
// results below 2^-126 flush to zero
__device__ __forceinline__ float exp2_neg(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kRescaleLog2 = 8.f;   // lazy softmax rescale: keep exp2(s - m) <= 2^8

// Where an item's keys are: chunk [t0, t1) of the row's visible keys, of which
// [nb, t1) are this call's appended rows (taken from LDS, not the cache).
// PG (paged cache): the chunk's keys lie in pages t0 / psz .. (t1 - 1) / psz, at
// most 64 of them (a chunk holds at most 1024 keys, a page at least 16); lane j
// holds the id of the j-th (lanes past the chunk: the table row's last entry),
// an id outside the pool replaced by page 0 so that every address stays in the
// pool; pbad: the chunk needs such a page.  kvrow0 is then the kv head's first
// row inside a page.
struct ItemGeom {
  int L, r_off, t0, t1, nb, n_new, tw, nsteps, last_row;
  size_t kvrow0;
  int slot, pg;
  bool pbad;
};

template <bool PG = false>
__device__ __forceinline__ ItemGeom item_geom(const LayerArgs &A, const Item &it, int4 rin) {
  // rin: slot, committed length, visible keys, block offset (uniform over the workgroup)
  rin = make_int4(__builtin_amdgcn_readfirstlane(rin.x), __builtin_amdgcn_readfirstlane(rin.y),
                  __builtin_amdgcn_readfirstlane(rin.z), __builtin_amdgcn_readfirstlane(rin.w));
  ItemGeom g;
  g.L = rin.y;
  g.r_off = rin.w;
  g.t0 = it.c * A.split;
  g.t1 = min(g.t0 + A.split, rin.z);
  g.nb = max(g.t0, g.L);
  g.n_new = max(0, g.t1 - g.nb);
  g.slot = rin.x;
  if constexpr (PG) {
    const int lane = lane_id();
    const int p0 = g.t0 >> A.plog, npg = ((g.t1 - 1) >> A.plog) - p0 + 1;
    const int pid = A.ptab[(size_t)rin.x * A.pps + min(p0 + lane, A.pps - 1)];
    const bool ok = (unsigned)pid < (unsigned)A.npages;
    g.pg = ok ? pid : 0;
    g.pbad = __any(lane < npg && !ok) != 0;
    g.kvrow0 = (size_t)it.g * A.psz;
  } else {
    g.pg = 0;
    g.pbad = false;
    g.kvrow0 = ((size_t)rin.x * A.nkv + it.g) * A.capacity;
  }
  g.tw = g.t0 + wave_id() * 8;
  g.nsteps = g.tw < g.t1 ? (g.t1 - g.tw + 31) / 32 : 0;
  g.last_row = max(min(g.t1, g.L) - 1, 0);
  return g;
}
template <bool PG = false>
__device__ __forceinline__ ItemGeom item_geom(const LayerArgs &A, const Item &it, const int4 *rinfo) {
  return item_geom<PG>(A, it, rinfo[it.row]);
}

// The K and V registers of two 32-key steps of an item (lane: one key row of
// its wave's 8, dims [8 kl, 8 kl + 8) and [64 + 8 kl, 64 + 8 kl + 8)).
struct KVRegs {
  uint4 a0, a1, a2, a3, b0, b1, b2, b3;
};

// Steps of 8 keys per wave, two steps in flight while one is computed.  Every
// load is unconditional (rows clamped to the chunk's last committed row, so
// the loads past the chunk hit lines this item already fetched) so the
// compiler can count the loads in flight exactly; lanes past the chunk get
// weight 0.  Each 16-byte load instruction of a wave covers whole 128-byte lines.
// PG: the key row's page comes from the lane that holds it (a row clamped below
// the chunk takes the chunk's first page: its value is never used), so every
// address is inside the pool.
template <bool PG = false>
__device__ __forceinline__ void kv_load_step(const LayerArgs &A, const ItemGeom &g, uint4 (&r)[4], int i) {
  const int lane = lane_id(), kl = lane & 7, kr = lane >> 3;
  if constexpr (PG) {
    const int row = min(g.tw + 32 * i + kr, g.last_row);
    const int j = min(max((row >> A.plog) - (g.t0 >> A.plog), 0), kWave - 1);
    const int page = __shfl(g.pg, j, kWave);
    const size_t e = ((size_t)page * A.nkv * A.psz + g.kvrow0 + (row & (A.psz - 1))) * kHeadDim + kl * 8;
    r[0] = ld16(A.kc + e);
    r[1] = ld16(A.kc + e + 64);
    r[2] = ld16(A.vc + e);
    r[3] = ld16(A.vc + e + 64);
    return;
  }
  const uint32_t region = (uint32_t)A.capacity * kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(A.kc + g.kvrow0 * kHeadDim, region);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(A.vc + g.kvrow0 * kHeadDim, region);
  const uint32_t off = (uint32_t)min(g.tw + 32 * i + kr, g.last_row) * (kHeadDim * 2) + kl * 16;
  r[0] = ld_buf(Kr, off);
  r[1] = ld_buf(Kr, off + 128);
  r[2] = ld_buf(Vr, off);
  r[3] = ld_buf(Vr, off + 128);
}

template <bool PG = false>
__device__ __forceinline__ void attn_item_loads(const LayerArgs &A, const Item &it, const int4 *rinfo, KVRegs &P) {
  const ItemGeom g = item_geom<PG>(A, it, rinfo);
  uint4 a[4], b[4];
  kv_load_step<PG>(A, g, a, 0);
  kv_load_step<PG>(A, g, b, 1);
  P = KVRegs{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The q vectors an item reads from this call's projection: its GROUP q heads
// (this lane's 16 dims of each) and their norm partials; requested, not waited for.
template <int GROUP>
struct QLoads {
  float4 v[GROUP][4], p[GROUP][2];
};

template <int GROUP>
__device__ __forceinline__ void q_loads(const LayerArgs &A, int row, int g, QLoads<GROUP> &Q) {
  const int kl = lane_id() & 7;
  const int d0 = 8 * kl, d1 = 64 + 8 * kl;
  const __amdgpu_buffer_rsrc_t Qr = rsrc_of(A.qkv + (size_t)row * A.nqkv, (uint32_t)A.nqkv * 4);
  const __amdgpu_buffer_rsrc_t Sr = rsrc_of(A.ssq + (size_t)row * (A.nq + A.nkv) * kTilesPerHead,
                                            (uint32_t)(A.nq + A.nkv) * kTilesPerHead * 4);
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    const uint32_t h = g * GROUP + j;
    Q.v[j][0] = ld_dev4(Qr, (h * kHeadDim + d0) * 4);
    Q.v[j][1] = ld_dev4(Qr, (h * kHeadDim + d0 + 4) * 4);
    Q.v[j][2] = ld_dev4(Qr, (h * kHeadDim + d1) * 4);
    Q.v[j][3] = ld_dev4(Qr, (h * kHeadDim + d1 + 4) * 4);
    Q.p[j][0] = ld_dev4(Sr, h * kTilesPerHead * 4);
    Q.p[j][1] = ld_dev4(Sr, (h * kTilesPerHead + 4) * 4);
  }
}

// q of the GROUP heads: rotated, gained projection / rms, times log2(e)/sqrt(d)
template <int GROUP>
__device__ __forceinline__ void q_scale(const LayerArgs &A, const QLoads<GROUP> &Q, float (&q)[GROUP][16]) {
  const float qs = kLog2e * rsqrtf((float)kHeadDim);
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    const float sc = inv_rms_of(A, Q.p[j][0], Q.p[j][1]) * qs;
#pragma unroll
    for (int h2 = 0; h2 < 4; ++h2) {
      q[j][4 * h2 + 0] = Q.v[j][h2].x * sc;
      q[j][4 * h2 + 1] = Q.v[j][h2].y * sc;
      q[j][4 * h2 + 2] = Q.v[j][h2].z * sc;
      q[j][4 * h2 + 3] = Q.v[j][h2].w * sc;
    }
  }
}

// One lane's two dims of an appended row as the cache stores them: k
// normalised with its head's partial sums, v raw, both rounded to 16 bits.
template <int DT>
__device__ __forceinline__ void fresh_pair(const LayerArgs &A, float4 k4, float4 v4, float4 kp0, float4 kp1,
                                           uint32_t &kb, uint32_t &vb) {
  const int lane = lane_id();
  const float2 kx = (lane & 1) ? make_float2(k4.z, k4.w) : make_float2(k4.x, k4.y);
  const float2 vx = (lane & 1) ? make_float2(v4.z, v4.w) : make_float2(v4.x, v4.y);
  const float inv = inv_rms_of(A, kp0, kp1);
  kb = (uint32_t)rne16<DT>(kx.x * inv) | ((uint32_t)rne16<DT>(kx.y * inv) << 16);
  vb = (uint32_t)rne16<DT>(vx.x) | ((uint32_t)rne16<DT>(vx.y) << 16);
}

// The key stream of an item whose first two steps are in ra, rb (the rest are
// loaded here) and whose appended rows, if any, are in knew/vnew: online
// softmax per wave, the 4 waves combined in LDS, the partial (m, l, acc) of
// each q head stored (device-coherent when COH: merged within the dispatch).
template <int DT, int GROUP, bool COH, int NP, bool PG = false>
__device__ __forceinline__ void attn_stream(const LayerArgs &A, const ItemGeom &G, int row, int g, int c,
                                            const float (&q)[GROUP][16], const uint16_t *knew,
                                            const uint16_t *vnew, AttnShared<GROUP> &S, uint4 (&r)[NP][4]) {
  static_assert(NP == 2 || NP == 4, "two or four steps loaded ahead");
  uint4 (&ra)[4] = r[0];
  uint4 (&rb)[4] = r[1];
  const int wave = wave_id(), lane = lane_id();
  const int kl = lane & 7, kr = lane >> 3;
  const int d0 = 8 * kl, d1 = 64 + 8 * kl;
  const int L = G.L, t1 = G.t1, nb = G.nb, tw = G.tw, nsteps = G.nsteps;
  auto load_step = [&](uint4 (&r)[4], int i) __attribute__((always_inline)) { kv_load_step<PG>(A, G, r, i); };

  float m[GROUP], l[GROUP], acc[GROUP][16];
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  }
  // Online softmax with a lazy reference: p = 2^(s - m) against a per-wave
  // reference m that moves only when some score passes it by more than 2^8
  // (a wave vote), so most steps skip the rescale of l and acc.
  auto compute_step = [&](const uint4 (&r)[4], int i, bool with_new) __attribute__((always_inline)) {
    const int t = tw + 32 * i + kr;
    const bool valid = t < t1;
    uint4 k0 = r[0], k1 = r[1], v0 = r[2], v1 = r[3];
    if (with_new) {
      const bool fresh = valid && t >= L;
      const int ni = fresh ? t - nb : 0;
      // LDS-typed reads: a select between them and the registers stays a value select
      const uint16_t *kn = knew + ni * kHeadDim, *vn = vnew + ni * kHeadDim;
      const uint4 a0 = lds_ld16(kn + d0), a1 = lds_ld16(kn + d1);
      const uint4 b0 = lds_ld16(vn + d0), b1 = lds_ld16(vn + d1);
      if (fresh) {
        k0 = a0; k1 = a1; v0 = b0; v1 = b1;
      }
    }
    if (!valid) k0 = k1 = v0 = v1 = make_uint4(0u, 0u, 0u, 0u);   // no stale inf/NaN bits
    float kf[16], vf[16];
    unpack8<DT>(k0, kf);
    unpack8<DT>(k1, kf + 8);
    unpack8<DT>(v0, vf);
    unpack8<DT>(v1, vf + 8);
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) s += q[j][e] * kf[e];
      s = sum8(s);
      s = valid ? s : -INFINITY;
      if (__any(s > m[j] + kRescaleLog2)) {
        // new reference: the wave max of this step (row_mirror pairs the two key
        // groups of a 16-lane row; readlane combines the four rows)
        float smax = fmaxf(s, dpp<kRowMirror>(s));
        smax = fmaxf(fmaxf(readlane(smax, 0), readlane(smax, 16)), fmaxf(readlane(smax, 32), readlane(smax, 48)));
        const float mn = fmaxf(m[j], smax);
        const float corr = exp2_neg(m[j] - mn);   // 0 on the first step (m = -inf)
        m[j] = mn;
        l[j] *= corr;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] *= corr;
      }
      const float p = valid ? exp2_neg(s - m[j]) : 0.f;
      l[j] += p;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] += p * vf[e];
    }
  };
  // The NP steps loaded by the caller first; after them two steps in flight
  // while one is computed.  No load is issued for a step past the item but the
  // odd one of the last pair (an outstanding load would hold the barrier below).
  auto run = [&](bool with_new) __attribute__((always_inline)) {
    int i = 0;
    if constexpr (NP == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k < nsteps) compute_step(r[k], k, with_new);
      if (nsteps <= 4) return;
      i = 4;
      load_step(ra, 4);
      load_step(rb, 5);
    }
    for (; i + 2 < nsteps; i += 2) {
      compute_step(ra, i, with_new);
      load_step(ra, i + 2);
      compute_step(rb, i + 1, with_new);
      load_step(rb, i + 3);
    }
    if (i < nsteps) compute_step(ra, i, with_new);
    if (i + 1 < nsteps) compute_step(rb, i + 1, with_new);
  };
  if (G.n_new == 0) run(false);
  else run(true);
  // combine the 8 key groups of the wave (lanes with equal kl), then the waves
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    l[j] = sum_stride8(l[j]);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = sum_stride8(acc[j][e]);
  }
  if (kr == 1) {   // lanes 8..15 hold the totals
#pragma unroll
    for (int j = 0; j < GROUP; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        S.acc[wave][j][d0 + e] = acc[j][e];
        S.acc[wave][j][d1 + e] = acc[j][8 + e];
      }
  }
  if (lane == 8) {
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
      const float sc = S.m[w][j] == -INFINITY ? 0.f : exp2_neg(S.m[w][j] - M);
      a += sc * S.acc[w][j][d];
      ls += sc * S.l[w][j];
    }
    stx<COH>(pbase + j * kPartStride + d, a);
    if (d == 0) {
      stx<COH>(pbase + j * kPartStride + 128, M);
      stx<COH>(pbase + j * kPartStride + 129, ls);
    }
  }
  __syncthreads();
}

// One item, its first two steps already loaded into P; its partial is merged by
// another workgroup of this same dispatch.
template <int DT, int GROUP, bool COH, bool PG = false>
__device__ __forceinline__ void attn_item(const LayerArgs &A, const Item &it, const int4 *rinfo, uint16_t *knew, uint16_t *vnew,
                          AttnShared<GROUP> &S, const KVRegs &P) {
  const int wave = wave_id(), lane = lane_id();
  const int row = it.row, g = it.g;
  const ItemGeom G = item_geom<PG>(A, it, rinfo);
  if constexpr (PG) {
    if (G.pbad && threadIdx.x == 0 && A.status) atomicOr(A.status, kStatusBadPage);
  }
  const int L = G.L, r_off = G.r_off, nb = G.nb, n_new = G.n_new;
  uint4 rr[2][4] = {{P.a0, P.a1, P.a2, P.a3}, {P.b0, P.b1, P.b2, P.b3}};

  // Everything the item reads from this call's projection is loaded up front in
  // one batch: its q heads, their norm partials, and for a chunk holding
  // appended rows the k/v rows and k partials.
  const uint32_t row_bytes = (uint32_t)A.nqkv * 4;
  QLoads<GROUP> Q;
  q_loads<GROUP>(A, row, g, Q);
  // appended rows (positions nb .. t1-1 = rows nb - L .. of this sequence): wave w
  // takes rows w, w + 4, ...; lane l holds dims 2l, 2l + 1
  const int n_mine = n_new > wave ? (n_new - wave + 3) / 4 : 0;
  for (int i0 = 0; i0 < n_mine; i0 += 2) {
    float4 k4[2], v4[2], kp[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = wave + 4 * (i0 + u);
      const int rrow = row - r_off + (nb + min(i, n_new - 1) - L);
      const __amdgpu_buffer_rsrc_t Rr = rsrc_of(A.qkv + (size_t)rrow * A.nqkv, row_bytes);
      k4[u] = ld_dev4(Rr, ((A.nq + g) * kHeadDim + 2 * (lane & ~1)) * 4);
      v4[u] = ld_dev4(Rr, ((A.nq + A.nkv + g) * kHeadDim + 2 * (lane & ~1)) * 4);
      const __amdgpu_buffer_rsrc_t Pr = rsrc_of(A.ssq + (size_t)rrow * (A.nq + A.nkv) * kTilesPerHead,
                                                (uint32_t)(A.nq + A.nkv) * kTilesPerHead * 4);
      kp[u][0] = ld_dev4(Pr, (A.nq + g) * kTilesPerHead * 4);
      kp[u][1] = ld_dev4(Pr, ((A.nq + g) * kTilesPerHead + 4) * 4);
    }
    const int own = L + r_off - nb;   // the row's own appended row (position L + r_off), if in the chunk
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = wave + 4 * (i0 + u);
      if (i >= n_new) break;
      uint32_t kb, vb;
      fresh_pair<DT>(A, k4[u], v4[u], kp[u][0], kp[u][1], kb, vb);
      reinterpret_cast<uint32_t *>(knew + i * kHeadDim)[lane] = kb;
      reinterpret_cast<uint32_t *>(vnew + i * kHeadDim)[lane] = vb;
      if (i == own) {   // every row also stores its own appended row in the cache
        if constexpr (PG) {
          // position nb + i = L + r_off: row (nb + i) % psz of the chunk's page (nb + i) / psz
          if (!G.pbad) {
            const int t = nb + i;
            const int page = __shfl(G.pg, (t >> A.plog) - (G.t0 >> A.plog), kWave);
            const size_t off = ((size_t)page * A.nkv * A.psz + G.kvrow0 + (t & (A.psz - 1))) * kHeadDim;
            reinterpret_cast<uint32_t *>(A.kc + off)[lane] = kb;
            reinterpret_cast<uint32_t *>(A.vc + off)[lane] = vb;
          }
        } else {
          const size_t off = (G.kvrow0 + nb + i) * kHeadDim;
          reinterpret_cast<uint32_t *>(A.kc + off)[lane] = kb;
          reinterpret_cast<uint32_t *>(A.vc + off)[lane] = vb;
        }
      }
    }
  }
  float q[GROUP][16];
  q_scale<GROUP>(A, Q, q);
  if (n_new > 0) __syncthreads();
  attn_stream<DT, GROUP, true, 2, PG>(A, G, row, g, it.c, q, knew, vnew, S, rr);
}

// ---------------------------------------------------------------- merge
//
// att[row][h] = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, M = max_c m_c,
// summed in chunk order (deterministic: never in the order the chunks
// finished).  Both merge sites (the last item of a (row, g) within the
// attention dispatch, or the o_proj kernel of the few-row path) run
// merge_column on the same partials, so every dispatch mode gives the same bits.

// Partial (m, l) and acc of chunk c of one float4 column: P(c, ml, av).
// ml0/av0 hold chunks [0, CB), requested by the caller; later chunks are
// requested here CB at a time.
template <int CB, class P>
__device__ __forceinline__ float4 merge_column(int nch, const float2 (&ml0)[CB], const float4 (&av0)[CB], P part) {
  // chunks past nch weigh nothing, by selects rather than branches (their slots
  // may hold an older call's values), so the terms of a batch schedule freely
  auto batch_max = [&](const float2 (&ml)[CB], int c0) __attribute__((always_inline)) {
    float x[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) x[c] = c0 + c < nch ? ml[c].x : -INFINITY;
#pragma unroll
    for (int w = 1; w < CB; w *= 2)
#pragma unroll
      for (int c = 0; c + w < CB; c += 2 * w) x[c] = fmaxf(x[c], x[c + w]);
    return x[0];
  };
  float M = batch_max(ml0, 0);
  for (int c0 = CB; c0 < nch; c0 += CB) {
    float2 ml[CB];
    float4 av;
#pragma unroll
    for (int u = 0; u < CB; ++u) part(c0 + u, ml[u], av, false);
    M = fmaxf(M, batch_max(ml, c0));
  }
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  auto add = [&](float2 ml, float4 av, bool ok) __attribute__((always_inline)) {
    const float w = ok ? exp2_neg(ml.x - M) : 0.f;
    const float l = ok ? ml.y : 0.f;
    const float4 a = ok ? av : make_float4(0.f, 0.f, 0.f, 0.f);
    den += w * l;
    num.x += w * a.x;
    num.y += w * a.y;
    num.z += w * a.z;
    num.w += w * a.w;
  };
#pragma unroll
  for (int c = 0; c < CB; ++c) add(ml0[c], av0[c], c < nch);
  for (int c0 = CB; c0 < nch; c0 += CB) {
    float2 ml[CB];
    float4 av[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) part(c0 + u, ml[u], av[u], true);
#pragma unroll
    for (int u = 0; u < CB; ++u) add(ml[u], av[u], c0 + u < nch);
  }
  const float inv = 1.0f / den;
  return make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
}

// chunk partials of one column read device-coherently (stored by other
// workgroups of this dispatch); past nch the buffer range reads zeros
struct PartCoherent {
  __amdgpu_buffer_rsrc_t R;   // the (row, kv head)'s partials: uniform over the workgroup
  uint32_t cs, head, col;     // bytes per chunk, byte offsets of the q head and of the column
  __device__ __forceinline__ void operator()(int c, float2 &ml, float4 &av, bool with_av) const {
    const float4 v = ld_dev4(R, c * cs + head + 128 * 4);
    ml = make_float2(v.x, v.y);
    if (with_av) av = ld_dev4(R, c * cs + head + col);
  }
};

// The last item of (row, g) to finish merges its GROUP heads: thread t <
// GROUP * 32 takes float4 column t of the GROUP x 128 outputs.
template <int DT, int GROUP, bool COH>
__device__ void merge_group(const LayerArgs &A, int row, int g, int nch, AttnShared<GROUP> &S) {
  // (uniform over the workgroup: scalar registers for the resources built from them)
  row = __builtin_amdgcn_readfirstlane(row);
  g = __builtin_amdgcn_readfirstlane(g);
  nch = __builtin_amdgcn_readfirstlane(nch);
  constexpr int CB = 8;
  const int t = threadIdx.x;
  if (t < GROUP * 32) {
    const int j = t / 32, d = (t % 32) * 4;
    // the head j of this thread goes into the offset, so the resource stays uniform
    const float *p0 = A.part + (((size_t)row * A.nkv + g) * kMaxChunks) * GROUP * kPartStride;
    const uint32_t cs = (uint32_t)GROUP * kPartStride * 4;
    const PartCoherent P{rsrc_of(p0, (uint32_t)nch * cs), cs, (uint32_t)j * kPartStride * 4, (uint32_t)d * 4};
    float2 ml[CB];
    float4 av[CB];
#pragma unroll
    for (int u = 0; u < CB; ++u) P(u, ml[u], av[u], true);
    const float4 o = merge_column<CB>(nch, ml, av, P);
    const size_t col = (size_t)(g * GROUP + j) * kHeadDim + d;
    const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) stx<COH>(A.att + (size_t)row * A.nq * kHeadDim + col + e, ov[e]);
    if (A.mfma) {   // tiled [plane][col / 32][row][32]: one MFMA operand load reads 1 KB contiguously
      const size_t plane = (size_t)(A.nq * kHeadDim / 32) * A.rows * 32;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const size_t idx = (((col + e) / 32) * A.rows + row) * 32 + (col + e) % 32;
        const uint16_t hi = rne16<DT>(ov[e]);
        A.att_hl[idx] = hi;
        A.att_hl[plane + idx] = rne16<DT>(ov[e] - cvt16<DT>(hi));
      }
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(A.mctr + (size_t)row * A.nkv + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
}

struct Pending {
  int row, g, nch;
  uint32_t old;     // counter value before this item's increment (thread 0 only)
};

// this item's partial is stored (by every thread): count it
__device__ __forceinline__ Pending signal_item(const LayerArgs &A, const Item &it) {
  wait_mem();
  __syncthreads();
  Pending p{it.row, it.g, it.nch, 0u};
  if (threadIdx.x == 0)
    p.old = __hip_atomic_fetch_add(A.mctr + (size_t)it.row * A.nkv + it.g, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  return p;
}

template <int DT, int GROUP, bool COH>
__device__ __forceinline__ void resolve(const LayerArgs &A, const Pending &p, AttnShared<GROUP> &S) {
  if (threadIdx.x == 0) S.flag = p.old == (uint32_t)(p.nch - 1);
  __syncthreads();
  if (S.flag) merge_group<DT, GROUP, COH>(A, p.row, p.g, p.nch, S);
}

template <int DT, int GROUP, bool COH, bool PG = false>
__device__ __forceinline__ void attention_phase(const LayerArgs &A, const int *pre, const int4 *rinfo, uint16_t *knew,
                                uint16_t *vnew, AttnShared<GROUP> &S, int first, int stride) {
  const int total = pre[A.rows];
  Pending pend{-1, 0, 0, 0u};
  for (int item = first; item < total; item += stride) {
    const Item it = decode_item(A, item, pre);
    KVRegs P;
    attn_item_loads<PG>(A, it, rinfo, P);
    attn_item<DT, GROUP, COH, PG>(A, it, rinfo, knew, vnew, S, P);
    const Pending now = signal_item(A, it);
    if (pend.row >= 0) resolve<DT, GROUP, COH>(A, pend, S);
    pend = now;
  }
  if (pend.row >= 0) resolve<DT, GROUP, COH>(A, pend, S);
}

// ---------------------------------------------------------------- phase C for many rows: equal key shares
//
// With many rows the attention work is the committed K/V stream.  The visible
// keys of all (row, kv head) pairs, concatenated in (row, g) order, are cut
// into equal shares, one per wave of a resident grid, so every wave streams
// the same number of keys whatever the length mix (no tail of long chunks).  A
// share holds one or more pieces (runs of keys of one (row, g)); a piece ends
// in a partial (m, l, acc) stored at slot (share index - share index of the
// (row, g)'s first key).  Waves work alone: no LDS traffic and no barrier after
// the prologue.  The loads run two 8-key steps ahead of the arithmetic, across
// piece boundaries.  Keys at or past the committed length are this call's
// appended rows: their k/v come from the projection (k normalised, both
// rounded to 16 bits as the cache stores them), and the piece of the
// sequence's last row writes them to the cache.  The last piece of a (row, g)
// to be counted merges the partials in slot order (deterministic).

// wave-uniform position of a wave's load or arithmetic stream
struct WCur {
  int row, g, t, te, grem;   // step keys [t, t + 8) of the piece [., te) of (row, g); keys of the share after te
  int P;                     // global index of key 0 of (row, g)
  int slot, L, nvis, roff;
};

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ void wcur_enter(WCur &c, const LayerArgs &A, const int *pre, const int4 *rinfo, int row,
                                           int g, int a, int keys) {
  const int4 ri = rinfo[row];
  c.row = row;
  c.g = g;
  c.t = a;
  c.slot = rfl(ri.x);
  c.L = rfl(ri.y);
  c.nvis = rfl(ri.z);
  c.roff = rfl(ri.w);
  c.P = rfl(pre[row]) + g * c.nvis;
  const int len = min(c.nvis - a, keys);
  c.te = a + len;
  c.grem = keys - len;
}

// next step: 1 in the same piece, 2 in a new piece, 0 past the share (unchanged)
__device__ __forceinline__ int wcur_next(WCur &c, const LayerArgs &A, const int *pre, const int4 *rinfo) {
  if (c.t + 8 < c.te) {
    c.t += 8;
    return 1;
  }
  if (c.grem == 0) return 0;
  int row = c.row, g = c.g + 1;
  if (g == A.nkv) {
    g = 0;
    do {
      ++row;
    } while (row < A.rows - 1 && rfl(rinfo[row].z) == 0);
    if (rfl(rinfo[row].z) == 0) return 0;   // (no keys left: the share ends)
  }
  wcur_enter(c, A, pre, rinfo, row, g, 0, c.grem);
  return 2;
}

// K and V of one step: lane = key t + (lane >> 3), dims [8 kl, 8 kl + 8) and [64 + 8 kl, ..)
// (kl = lane & 7); rows clamped to the piece's last committed key, so past
// the piece the loads hit lines already fetched.  NT: the call reads each
// cached row once (one row per sequence), so the stream carries the
// nontemporal hint; rows of a verify block read their sequence's rows again
// and keep plain loads.
// F8: the cache holds E4M3 codes (128-byte rows); lane kl takes dims
// [16 kl, 16 kl + 16) with one 16-byte load, so a wave's load covers 8 whole lines.
// Entry `pidx` of slot `slot`'s page table, both wave-uniform: read through the
// scalar cache, so that waiting for it never waits on the K/V loads in flight.
__device__ __forceinline__ int page_entry(const LayerArgs &A, int slot, int pidx) {
  typedef const __attribute__((address_space(4))) int32_t *ctab_t;
  return ((ctab_t)A.ptab)[(size_t)slot * A.pps + pidx];
}

// PG (paged cache): the step's rows lie in at most two pages (a page holds at
// least 16 rows), whose ids are read as wave-uniform values; each lane takes
// its row's.  An id outside the pool is replaced by page 0 (the return value
// says so), so every address stays in the pool.
template <bool NT, bool F8, bool PG = false>
__device__ __forceinline__ bool wstep_load(const LayerArgs &A, const WCur &c, uint4 (&r)[4]) {
  const int lane = lane_id(), kl = lane & 7, kr = lane >> 3;
  if constexpr (PG) {
    static_assert(!F8, "paged caches hold 16-bit rows");
    const int last = max(min(rfl(c.te), rfl(c.L)) - 1, 0);
    const int slot = rfl(c.slot), t = rfl(c.t);
    const int ia = min(t, last) >> A.plog, ib = min(t + 7, last) >> A.plog;
    const int pa = page_entry(A, slot, ia), pb = page_entry(A, slot, ib);
    const bool oka = (unsigned)pa < (unsigned)A.npages, okb = (unsigned)pb < (unsigned)A.npages;
    const int row = min(t + kr, last);
    const int page = (row >> A.plog) == ia ? (oka ? pa : 0) : (okb ? pb : 0);
    const size_t e = (((size_t)page * A.nkv + rfl(c.g)) * A.psz + (row & (A.psz - 1))) * kHeadDim + kl * 8;
    r[0] = NT ? ld16_stream(A.kc + e) : ld16(A.kc + e);
    r[1] = NT ? ld16_stream(A.kc + e + 64) : ld16(A.kc + e + 64);
    r[2] = NT ? ld16_stream(A.vc + e) : ld16(A.vc + e);
    r[3] = NT ? ld16_stream(A.vc + e + 64) : ld16(A.vc + e + 64);
    return !(oka && okb);
  }
  constexpr uint32_t RB = F8 ? kHeadDim : kHeadDim * 2;   // bytes per cached row
  // (the cursor is wave-uniform; readfirstlane keeps the resources in scalar registers)
  const size_t base = ((size_t)rfl(c.slot) * A.nkv + rfl(c.g)) * A.capacity * RB;
  const uint32_t region = (uint32_t)A.capacity * RB;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(reinterpret_cast<const unsigned char *>(A.kc) + base, region);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(reinterpret_cast<const unsigned char *>(A.vc) + base, region);
  const int last = max(min(rfl(c.te), rfl(c.L)) - 1, 0);
  if constexpr (F8) {   // dims [16 kl, 16 kl + 16): one 16-byte load each for K and V
    const uint32_t off = (uint32_t)min(rfl(c.t) + kr, last) * RB + kl * 16;
    const uint4 a = NT ? ld_buf_nt(Kr, off) : ld_buf(Kr, off);
    const uint4 e = NT ? ld_buf_nt(Vr, off) : ld_buf(Vr, off);
    r[0] = make_uint4(a.x, a.y, 0u, 0u);
    r[1] = make_uint4(a.z, a.w, 0u, 0u);
    r[2] = make_uint4(e.x, e.y, 0u, 0u);
    r[3] = make_uint4(e.z, e.w, 0u, 0u);
  } else {
    const uint32_t off = (uint32_t)min(rfl(c.t) + kr, last) * RB + kl * 16;
    r[0] = NT ? ld_buf_nt(Kr, off) : ld_buf(Kr, off);
    r[1] = NT ? ld_buf_nt(Kr, off + 128) : ld_buf(Kr, off + 128);
    r[2] = NT ? ld_buf_nt(Vr, off) : ld_buf(Vr, off);
    r[3] = NT ? ld_buf_nt(Vr, off + 128) : ld_buf(Vr, off + 128);
  }
  return false;
}

// One lane's 8 dims of an appended row, 16-bit as stored: k normalised with
// its head's partial sums, v raw.
template <int DT>
__device__ __forceinline__ uint4 round8(float4 a, float4 b, float sc) {
  uint4 u;
  u.x = (uint32_t)rne16<DT>(a.x * sc) | ((uint32_t)rne16<DT>(a.y * sc) << 16);
  u.y = (uint32_t)rne16<DT>(a.z * sc) | ((uint32_t)rne16<DT>(a.w * sc) << 16);
  u.z = (uint32_t)rne16<DT>(b.x * sc) | ((uint32_t)rne16<DT>(b.y * sc) << 16);
  u.w = (uint32_t)rne16<DT>(b.z * sc) | ((uint32_t)rne16<DT>(b.w * sc) << 16);
  return u;
}
template <int DT>
__device__ __forceinline__ uint4 round8(float4 a, float4 b) {
  uint4 u;
  u.x = (uint32_t)rne16<DT>(a.x) | ((uint32_t)rne16<DT>(a.y) << 16);
  u.y = (uint32_t)rne16<DT>(a.z) | ((uint32_t)rne16<DT>(a.w) << 16);
  u.z = (uint32_t)rne16<DT>(b.x) | ((uint32_t)rne16<DT>(b.y) << 16);
  u.w = (uint32_t)rne16<DT>(b.z) | ((uint32_t)rne16<DT>(b.w) << 16);
  return u;
}

// counted partial of a piece whose merge check waits for a later point
struct WPending {
  int row, g, np;
  uint32_t old;   // counter before this piece's increment (lane 0)
};

// Merge of the np partials of (row, g) by one wave: weights 2^(m_c - M) / sum,
// chunks in slot order.  Lane c < np holds piece c's (m, l); lane l's outputs
// are the float4 columns o = l + 64 q of the GROUP x 128 result.
template <int DT, int GROUP>
__device__ void merge_wave(const LayerArgs &A, int row, int g, int np) {
  constexpr int NPL = GROUP / 2;   // float4 outputs per lane
  const int lane = lane_id();
  const float *p0 = A.part + (((size_t)row * A.nkv + g) * kMaxChunks * GROUP) * kPartStride;
  const uint32_t cs = (uint32_t)GROUP * kPartStride * 4;   // bytes per piece
  const __amdgpu_buffer_rsrc_t R = rsrc_of(p0, (uint32_t)np * cs);
  float wn[GROUP];
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    const float4 ml = ld_dev4(R, lane * cs + (j * kPartStride + 128) * 4);   // zeros past np
    const float m = lane < np ? ml.x : -INFINITY;
    const float M = wave_max(m);
    const float w = (lane < np && m != -INFINITY) ? exp2_neg(m - M) : 0.f;
    const float tot = wave_sum(w * ml.y);
    wn[j] = w / tot;
  }
  float4 a[NPL];
#pragma unroll
  for (int q = 0; q < NPL; ++q) a[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int BATCH = 8;
  for (int c0 = 0; c0 < np; c0 += BATCH) {
    float4 v[BATCH][NPL];
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const int o = lane + 64 * q, j = o / 32, d = (o % 32) * 4;
        v[u][q] = ld_dev4(R, (c0 + u) * cs + (j * kPartStride + d) * 4);   // zeros past np
      }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = min(c0 + u, kWave - 1);
#pragma unroll
      for (int q = 0; q < NPL; ++q) {
        const int jl = (lane + 64 * q) / 32;   // head of this output: 2q or 2q + 1
        const float w0 = readlane(wn[(2 * q) % GROUP], c), w1 = readlane(wn[(2 * q + 1) % GROUP], c);
        const float w = c0 + u < np ? ((jl & 1) ? w1 : w0) : 0.f;
        a[q].x += w * v[u][q].x;
        a[q].y += w * v[u][q].y;
        a[q].z += w * v[u][q].z;
        a[q].w += w * v[u][q].w;
      }
    }
  }
  const size_t plane = (size_t)(A.nq * kHeadDim / 32) * A.rows * 32;
#pragma unroll
  for (int q = 0; q < NPL; ++q) {
    const int o = lane + 64 * q, j = o / 32, d = (o % 32) * 4;
    const size_t col = (size_t)(g * GROUP + j) * kHeadDim + d;
    const float av[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
    *reinterpret_cast<float4 *>(A.att + (size_t)row * A.nq * kHeadDim + col) = a[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {   // tiled [plane][col / 32][row][32] for the MFMA o_proj
      const size_t idx = (((col + e) / 32) * A.rows + row) * 32 + (col + e) % 32;
      const uint16_t hi = rne16<DT>(av[e]);
      A.att_hl[idx] = hi;
      A.att_hl[plane + idx] = rne16<DT>(av[e] - cvt16<DT>(hi));
    }
  }
  if (lane == 0) __hip_atomic_store(A.mctr + (size_t)row * A.nkv + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DT, int GROUP>
__device__ __forceinline__ void wresolve(const LayerArgs &A, const WPending &p) {
  if (p.row < 0) return;
  const uint32_t old = (uint32_t)__builtin_amdgcn_readlane((int)p.old, 0);
  if (old == (uint32_t)(p.np - 1)) merge_wave<DT, GROUP>(A, p.row, p.g, p.np);
}

template <int DT, int GROUP, bool NT, bool F8, bool PG = false>
__device__ __forceinline__ void attention_waves(const LayerArgs &A, const int *pre, const int4 *rinfo, int w, int W) {
  const int lane = lane_id(), kl = lane & 7, kr = lane >> 3;
  // a lane's 16 dims: [8 kl, 8 kl + 8) and [64 + 8 kl, ..) of a 256-byte 16-bit row (two whole
  // lines per key across the 8 lanes), or [16 kl, 16 kl + 16) of a 128-byte FP8 row (one line)
  const int d0 = F8 ? 16 * kl : 8 * kl, d1 = F8 ? 16 * kl + 8 : 64 + 8 * kl;
  const int T = pre[A.rows];
  const int S = max(T / W + 1, A.split);
  const long long s0l = (long long)w * S;
  if (s0l >= T) return;
  const int s0 = (int)s0l, s1 = min(s0 + S, T);
  // the (row, g) holding key s0
  int lo = 0, hi = A.rows;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= s0) lo = mid; else hi = mid;
  }
  const int off = s0 - pre[lo], nv0 = rinfo[lo].z;
  WCur lc;
  wcur_enter(lc, A, pre, rinfo, lo, off / nv0, off % nv0, s1 - s0);
  WCur cc = lc;
  // NS register sets in rotation: the loads of step i + NS - 1 are issued before
  // the arithmetic of step i.  An FP8 step is half the bytes of a 16-bit one, so
  // it keeps twice as many steps in flight (the same bytes in flight per wave).
  constexpr int NS = F8 ? 5 : 3;
  uint4 rs[NS][4];
  bool pbad = false;   // PG: a page id outside the pool was met (loads or this wave's appended rows)
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) {
    pbad |= wstep_load<NT, F8, PG>(A, lc, rs[i]);
    wcur_next(lc, A, pre, rinfo);
  }

  const float qs = kLog2e * rsqrtf((float)kHeadDim);
  const uint32_t row_bytes = (uint32_t)A.nqkv * 4;
  const uint32_t ssq_bytes = (uint32_t)(A.nq + A.nkv) * kTilesPerHead * 4;
  float q[GROUP][16], m[GROUP], l[GROUP], acc[GROUP][16];
  WPending pend{-1, 0, 0, 0u};

  // q of the GROUP heads of (row, g): rotated, gained projection / rms, times log2(e)/sqrt(d)
  auto begin_piece = [&]() {
    const int crow = rfl(cc.row), cg = rfl(cc.g);
    const __amdgpu_buffer_rsrc_t Qr = rsrc_of(A.qkv + (size_t)crow * A.nqkv, row_bytes);
    const __amdgpu_buffer_rsrc_t Sr = rsrc_of(A.ssq + (size_t)crow * (A.nq + A.nkv) * kTilesPerHead, ssq_bytes);
    float4 qv[GROUP][4], qp[GROUP][2];
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      const uint32_t h = cg * GROUP + j;
      qv[j][0] = ld_dev4(Qr, (h * kHeadDim + d0) * 4);
      qv[j][1] = ld_dev4(Qr, (h * kHeadDim + d0 + 4) * 4);
      qv[j][2] = ld_dev4(Qr, (h * kHeadDim + d1) * 4);
      qv[j][3] = ld_dev4(Qr, (h * kHeadDim + d1 + 4) * 4);
      qp[j][0] = ld_dev4(Sr, h * kTilesPerHead * 4);
      qp[j][1] = ld_dev4(Sr, (h * kTilesPerHead + 4) * 4);
    }
    // an FP8 cache's K scale is folded into q (scores = (s_k q) . code values)
    const float ksc = F8 ? A.ksc[cg] : 1.f;
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      const float sc = inv_rms_of(A, qp[j][0], qp[j][1]) * qs * ksc;
#pragma unroll
      for (int h2 = 0; h2 < 4; ++h2) {
        q[j][4 * h2 + 0] = qv[j][h2].x * sc;
        q[j][4 * h2 + 1] = qv[j][h2].y * sc;
        q[j][4 * h2 + 2] = qv[j][h2].z * sc;
        q[j][4 * h2 + 3] = qv[j][h2].w * sc;
      }
      m[j] = -INFINITY;
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    }
  };

  // the piece of `c` is complete: partial to its slot, then count it
  auto finish_piece = [&](const WCur &c) {
    // an FP8 cache's V scale multiplies the weighted sum of code values
    const float vsc = F8 ? A.vsc[rfl(c.g)] : 1.f;
    float v32[GROUP * 16];
#pragma unroll
    for (int j = 0; j < GROUP; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) v32[j * 16 + e] = acc[j][e] * vsc;
    float v16[GROUP * 8], v8[GROUP * 4], v4[GROUP * 2];
    rs_half<GROUP * 16, 32>(v32, v16);
    rs_half<GROUP * 8, 16>(v16, v8);
    rs_half<GROUP * 4, 8>(v8, v4);
    float lt[GROUP];
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      float x = l[j];
      x = xsum<32>(x);
      x = xsum<16>(x);
      x = xsum<8>(x);
      lt[j] = x;
    }
    const int first = c.P / S;
    const int pc = w - first;
    const int np = (c.P + c.nvis - 1) / S - first + 1;
    float *pb = A.part + ((((size_t)c.row * A.nkv + c.g) * kMaxChunks + pc) * GROUP) * kPartStride;
    const __amdgpu_buffer_rsrc_t R = rsrc_of(pb, (uint32_t)GROUP * kPartStride * 4);
    // this lane's values: v4[4 u .. 4 u + 3] = list entries base + 4 u, base from lane bits 5, 4, 3
    const int base = ((lane >> 5) & 1) * (GROUP * 8) + ((lane >> 4) & 1) * (GROUP * 4) + ((lane >> 3) & 1) * (GROUP * 2);
#pragma unroll
    for (int u = 0; u < GROUP / 2; ++u) {
      const int i = base + 4 * u, j = i / 16, e = i % 16;
      const int d = e < 8 ? d0 + e : d1 + e - 8;
      st_dev4(R, (j * kPartStride + d) * 4, make_float4(v4[4 * u], v4[4 * u + 1], v4[4 * u + 2], v4[4 * u + 3]));
    }
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < GROUP; ++j) st_dev4(R, (j * kPartStride + 128) * 4, make_float4(m[j], lt[j], 0.f, 0.f));
    }
    wait_mem();   // the partial is performed before it is counted
    const WPending prev = pend;
    pend.row = c.row;
    pend.g = c.g;
    pend.np = np;
    pend.old = 0u;
    if (lane == 0)
      pend.old = __hip_atomic_fetch_add(A.mctr + (size_t)c.row * A.nkv + c.g, 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    wresolve<DT, GROUP>(A, prev);
  };

  // one 8-key step of the arithmetic stream (online softmax with a lazy reference
  // as in the chunked path: rescale only when a score passes it by 2^8)
  auto step = [&](const uint4 (&r)[4]) {
    const int t = cc.t + kr;
    const bool valid = t < cc.te;
    uint4 k0 = r[0], k1 = r[1], v0 = r[2], v1 = r[3];
    if (cc.t + 8 > cc.L && cc.t < cc.te) {   // the step holds appended rows
      if (valid && t >= cc.L) {
        // resources at the sequence's first row (wave-uniform), the appended row by offset
        const int row0 = rfl(cc.row) - rfl(cc.roff), i = t - rfl(cc.L), cg = rfl(cc.g);
        const __amdgpu_buffer_rsrc_t Rr = rsrc_of(A.qkv + (size_t)row0 * A.nqkv, (uint32_t)(rfl(cc.roff) + 1) * row_bytes);
        const __amdgpu_buffer_rsrc_t Pr =
            rsrc_of(A.ssq + (size_t)row0 * (A.nq + A.nkv) * kTilesPerHead, (uint32_t)(rfl(cc.roff) + 1) * ssq_bytes);
        const uint32_t kh = i * row_bytes + (A.nq + cg) * kHeadDim * 4, vh = i * row_bytes + (A.nq + A.nkv + cg) * kHeadDim * 4;
        const uint32_t ph = i * ssq_bytes + (A.nq + cg) * kTilesPerHead * 4;
        const float4 ka = ld_dev4(Rr, kh + d0 * 4), kb = ld_dev4(Rr, kh + (d0 + 4) * 4);
        const float4 kc = ld_dev4(Rr, kh + d1 * 4), kd = ld_dev4(Rr, kh + (d1 + 4) * 4);
        const float4 va = ld_dev4(Rr, vh + d0 * 4), vb = ld_dev4(Rr, vh + (d0 + 4) * 4);
        const float4 vc = ld_dev4(Rr, vh + d1 * 4), vd = ld_dev4(Rr, vh + (d1 + 4) * 4);
        const float4 p0 = ld_dev4(Pr, ph);
        const float4 p1 = ld_dev4(Pr, ph + 16);
        const float inv = inv_rms_of(A, p0, p1);
        if constexpr (F8) {   // codes of value / scale, as the cache stores them
          const float ik = inv / A.ksc[cg], iv = 1.f / A.vsc[cg];
          k0 = make_uint4(pack4_e4m3(ka.x * ik, ka.y * ik, ka.z * ik, ka.w * ik),
                          pack4_e4m3(kb.x * ik, kb.y * ik, kb.z * ik, kb.w * ik), 0u, 0u);
          k1 = make_uint4(pack4_e4m3(kc.x * ik, kc.y * ik, kc.z * ik, kc.w * ik),
                          pack4_e4m3(kd.x * ik, kd.y * ik, kd.z * ik, kd.w * ik), 0u, 0u);
          v0 = make_uint4(pack4_e4m3(va.x * iv, va.y * iv, va.z * iv, va.w * iv),
                          pack4_e4m3(vb.x * iv, vb.y * iv, vb.z * iv, vb.w * iv), 0u, 0u);
          v1 = make_uint4(pack4_e4m3(vc.x * iv, vc.y * iv, vc.z * iv, vc.w * iv),
                          pack4_e4m3(vd.x * iv, vd.y * iv, vd.z * iv, vd.w * iv), 0u, 0u);
          if (t == cc.L + cc.roff) {   // every row stores its own appended row
            const size_t ro = (((size_t)cc.slot * A.nkv + cc.g) * A.capacity + t) * kHeadDim;
            unsigned char *kc8 = reinterpret_cast<unsigned char *>(A.kc), *vc8 = reinterpret_cast<unsigned char *>(A.vc);
            *reinterpret_cast<uint2 *>(kc8 + ro + d0) = make_uint2(k0.x, k0.y);
            *reinterpret_cast<uint2 *>(kc8 + ro + d1) = make_uint2(k1.x, k1.y);
            *reinterpret_cast<uint2 *>(vc8 + ro + d0) = make_uint2(v0.x, v0.y);
            *reinterpret_cast<uint2 *>(vc8 + ro + d1) = make_uint2(v1.x, v1.y);
          }
        } else {
          k0 = round8<DT>(ka, kb, inv);
          k1 = round8<DT>(kc, kd, inv);
          v0 = round8<DT>(va, vb);
          v1 = round8<DT>(vc, vd);
          if (t == cc.L + cc.roff) {   // every row stores its own appended row
            size_t ro = (((size_t)cc.slot * A.nkv + cc.g) * A.capacity + t) * kHeadDim;
            bool store = true;
            if constexpr (PG) {   // row t % psz of its page (skipped, and reported, for an id outside the pool)
              const int own = rfl(cc.L) + rfl(cc.roff);
              const int pg = page_entry(A, rfl(cc.slot), own >> A.plog);
              store = (unsigned)pg < (unsigned)A.npages;
              pbad |= !store;
              ro = (((size_t)(store ? pg : 0) * A.nkv + cc.g) * A.psz + (own & (A.psz - 1))) * kHeadDim;
            }
            if (store) {
              *reinterpret_cast<uint4 *>(A.kc + ro + d0) = k0;
              *reinterpret_cast<uint4 *>(A.kc + ro + d1) = k1;
              *reinterpret_cast<uint4 *>(A.vc + ro + d0) = v0;
              *reinterpret_cast<uint4 *>(A.vc + ro + d1) = v1;
            }
          }
        }
      }
    }
    {   // invalid lanes: score -inf (a select below) and v zeroed with a mask, not a
        // branch, so the loads of later steps stay in flight
      const uint32_t vm = valid ? 0xffffffffu : 0u;
      v0 = make_uint4(v0.x & vm, v0.y & vm, v0.z & vm, v0.w & vm);
      v1 = make_uint4(v1.x & vm, v1.y & vm, v1.z & vm, v1.w & vm);
    }
    float kf[16], vf[16];
    if constexpr (F8) {
      unpack8_e4m3(k0.x, k0.y, kf);
      unpack8_e4m3(k1.x, k1.y, kf + 8);
      unpack8_e4m3(v0.x, v0.y, vf);
      unpack8_e4m3(v1.x, v1.y, vf + 8);
    } else {
      unpack8<DT>(k0, kf);
      unpack8<DT>(k1, kf + 8);
      unpack8<DT>(v0, vf);
      unpack8<DT>(v1, vf + 8);
    }
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) s += q[j][e] * kf[e];
      s = sum8(s);
      s = valid ? s : -INFINITY;
      if (__any(s > m[j] + kRescaleLog2)) {
        float smax = fmaxf(s, dpp<kRowMirror>(s));
        smax = fmaxf(fmaxf(readlane(smax, 0), readlane(smax, 16)), fmaxf(readlane(smax, 32), readlane(smax, 48)));
        const float mn = fmaxf(m[j], smax);
        const float corr = exp2_neg(m[j] - mn);
        m[j] = mn;
        l[j] *= corr;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] *= corr;
      }
      const float p = valid ? exp2_neg(s - m[j]) : 0.f;
      l[j] += p;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] += p * vf[e];
    }
  };

  auto issue = [&](uint4 (&r)[4]) {
    pbad |= wstep_load<NT, F8, PG>(A, lc, r);
    wcur_next(lc, A, pre, rinfo);
  };
  // arithmetic of cc's step, then advance cc: false past the share
  auto advance = [&](const uint4 (&r)[4]) -> bool {
    step(r);
    const WCur old = cc;
    const int st = wcur_next(cc, A, pre, rinfo);
    if (st == 1) return true;
    finish_piece(old);
    if (st == 0) return false;
    begin_piece();
    return true;
  };
  begin_piece();
  for (;;) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      issue(rs[(i + NS - 1) % NS]);
      if (!advance(rs[i])) goto streamed;
    }
  }
streamed:
  wresolve<DT, GROUP>(A, pend);
  if constexpr (PG) {
    if (__any(pbad) && lane == 0 && A.status) atomicOr(A.status, kStatusBadPage);
  }
}

// ---------------------------------------------------------------- phase D: o_proj
//
// Same structure as phase A with the attention output as input, read from LDS
// (merged by this block) or from the workspace.
// rinfo: the rows' (slot, length, visible keys, offset) in LDS, or NULL to read
// the row table in the workspace
template <int DT, int KV, int RB, int RPW, bool COH>
__device__ __forceinline__ void oproj_tile(const LayerArgs &A, int tile, const uint4 (&wr)[RPW][KV], const int4 *rinfo) {
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
          const float *src = A.att + (size_t)row * K + (v * 64 + lane) * 8;
          if constexpr (COH) {
            const __amdgpu_buffer_rsrc_t R = rsrc_of(A.att + (size_t)row * K, (uint32_t)K * 4);
            const float4 f0 = ld_dev4(R, (v * 64 + lane) * 32), f1 = ld_dev4(R, (v * 64 + lane) * 32 + 16);
            x[r][v * 8 + 0] = f0.x; x[r][v * 8 + 1] = f0.y; x[r][v * 8 + 2] = f0.z; x[r][v * 8 + 3] = f0.w;
            x[r][v * 8 + 4] = f1.x; x[r][v * 8 + 5] = f1.y; x[r][v * 8 + 6] = f1.z; x[r][v * 8 + 7] = f1.w;
          } else {
            const float4 f0 = reinterpret_cast<const float4 *>(src)[0], f1 = reinterpret_cast<const float4 *>(src)[1];
            x[r][v * 8 + 0] = f0.x; x[r][v * 8 + 1] = f0.y; x[r][v * 8 + 2] = f0.z; x[r][v * 8 + 3] = f0.w;
            x[r][v * 8 + 4] = f1.x; x[r][v * 8 + 5] = f1.y; x[r][v * 8 + 6] = f1.z; x[r][v * 8 + 7] = f1.w;
          }
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
        const bool row_ok = rinfo ? rinfo[row].z > 0 : read_row_table<COH>(A, row).x != 0;
        if (!row_ok) val = __builtin_nanf("");
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
template <bool COH, bool MIX = false>
__device__ void advance_lengths(const LayerArgs &A) {
  for (int b = threadIdx.x; b < A.B; b += blockDim.x) {
    const int4 rec = read_row_table<COH>(A, seq_row0<MIX>(A, b));
    if (rec.x) {
      A.lens[rec.z] = rec.y + seq_rows<MIX>(A, b);
    } else if (A.status) {
      atomicOr(A.status, rec.w ? (uint32_t)ASR_STATUS_CAPACITY : kStatusBadSlot);
    }
  }
}

// ---------------------------------------------------------------- dataflow counters (one-dispatch path)
//
// The one-dispatch path orders its phases with counters in the workspace
// instead of grid barriers: a consumer waits only for the producers it reads.
//   flow[h]             projection tiles of head h (q heads, k heads, v heads) stored
//   flow[kFlowMerged]   (row, kv head) pairs merged into the attention output
//   flow[kFlowStarted]  workgroups started (their tickets give the call's epoch)
//   flow[kFlowLensRead] workgroups that have read the lengths
// Counters are never reset: every call adds the same amount to each of them
// (kTilesPerHead per head, kFlowMergeUnit merges, kFlowStartUnit starts and
// reads; the
// shortfall of a call is added up front by workgroup 0), so the call's epoch e,
// taken from a workgroup's own ticket on flow[kFlowStarted], gives every target:
// counter == (e + 1) * unit in the low bits that e determines.  Producers store
// with st_dev, wait for their stores, then bump the counter; consumers poll
// with ld_dev.  Every wait is bounded: on timeout the status bit is set and the
// workgroup stops (the call's outputs are then undefined and the workspace must
// be zeroed again).
constexpr int kFlowMerged = 120, kFlowStarted = 121, kFlowLensRead = 122;
constexpr uint32_t kFlowStartShift = 12;                    // unit 4096 >= any grid
constexpr uint32_t kFlowStartUnit = 1u << kFlowStartShift;
constexpr uint32_t kFlowMergeUnit = 32;                     // >= rows * nkv of the path (4 x 8)
constexpr uint32_t kFlowEpochBits = 32 - kFlowStartShift;   // epochs are known modulo 2^20

// target of a counter with `unit` per call at the end of epoch e, and the bits it determines
struct FlowTarget {
  uint32_t value, mask;
};
__device__ __forceinline__ FlowTarget flow_target(uint32_t e, uint32_t unit) {
  const uint32_t mask = (uint32_t)(((unsigned long long)unit << kFlowEpochBits) - 1);
  return FlowTarget{((e + 1) * unit) & mask, mask};
}

// thread 0 only
__device__ bool spin_until(const LayerArgs &A, const uint32_t *c, FlowTarget t) {
  if ((ld_dev(c) & t.mask) == t.value) return true;
  const long long start = wall_clock64();
  while ((ld_dev(c) & t.mask) != t.value) {
    __builtin_amdgcn_s_sleep(1);
    if (wall_clock64() - start > kBarrierTimeoutTicks) {
      if (A.status) atomicOr(A.status, (uint32_t)ASR_STATUS_SYNC_TIMEOUT);
      return false;
    }
  }
  return true;
}

__device__ bool wait_count(const LayerArgs &A, const uint32_t *c, FlowTarget t, int *s_ok) {
  if (threadIdx.x == 0) *s_ok = spin_until(A, c, t);
  __syncthreads();
  return *s_ok != 0;
}

// every thread's stores of this workgroup are performed: count them
__device__ __forceinline__ void signal_count(uint32_t *c) {
  wait_mem();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// an item reads the q heads of its kv group and, when its chunk holds this
// call's rows, their k and v heads
__device__ bool wait_item_inputs(const LayerArgs &A, const Item &it, const int4 *rinfo, int group, uint32_t e,
                                 int *s_ok) {
  if (threadIdx.x == 0) {
    const FlowTarget t = flow_target(e, kTilesPerHead);
    bool ok = true;
    for (int j = 0; j < group && ok; ++j) ok = spin_until(A, A.flow + it.g * group + j, t);
    const ItemGeom g = item_geom(A, it, rinfo);
    if (ok && g.n_new > 0)
      ok = spin_until(A, A.flow + A.nq + it.g, t) && spin_until(A, A.flow + A.nq + A.nkv + it.g, t);
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// ---------------------------------------------------------------- kernels

// ---------------------------------------------------------------- batched projections on MFMA
//
// For more than a few rows the projections are dense contractions and run on
// v_mfma_f32_16x16x32.  A block owns 16 output features and 16 (o_proj) or 64
// (QKV) input rows; its four waves split the contraction dimension in
// quarters, request every operand of their quarter at once (one memory round
// trip, no step-by-step dependence) and add their partial tiles in LDS.  fp32
// operands are split into two 16-bit terms (hi = rne(v), lo = rne(v - hi)),
// exact 16-bit operands are used as they are, so the products keep about twice
// the 16-bit precision.
//
// Blocks of one output-feature tile are placed on one XCD (workgroups go to the
// XCDs round-robin): the weight tile they share is fetched into that XCD's L2
// once.  The number of feature tiles is a multiple of 8.
struct TileMap {
  int col, row;   // feature tile, row tile
};
__device__ __forceinline__ TileMap tile_of(int b, int rtiles) {
  const int q = b / (8 * rtiles), rem = b - q * 8 * rtiles;
  return TileMap{q * 8 + rem % 8, rem / 8};
}

// o_proj steps per operand batch: all of a wave's quarter up to 16 steps, else an even split
constexpr int chunk_steps(int kq) {
  return kq <= 16 ? kq : (kq % 16 == 0 ? 16 : (kq % 12 == 0 ? 12 : (kq % 14 == 0 ? 14 : (kq % 10 == 0 ? 10 : 4))));
}

// QKV: out[n][o] = inv_rms(x_n) * sum_k (W[o][k] g_in[k]) x[n][k].  The weight
// times the input-norm gain is formed in fp32 (exact: two 16-bit factors) and
// split; x is the exact 16-bit operand; the sums of squares of x for inv_rms are
// accumulated from the same loads.  A block owns 16 features x 64 rows (four
// row tiles share each split weight step); the 16 features are 8 rotary pairs
// (t, t + 64) of one head, as in the vector path, with the same epilogue: gain
// and rotation of q/k pairs, partial sums of squares, v stored raw.
// LX (hidden 1024 and 2048, eight waves): per batch of four 32-wide steps, each
// wave loads its 64 rows x 256 bytes of x as whole 128-byte lines (four rows
// per instruction) into its own 16 KB LDS region and reads the operand layout
// back from there: the operand layout touches 16 rows per load, half a line
// each, and a CU keeps only so many lines in flight.  At hidden 2048 a wave's
// share takes two batches.
template <int DT, int KQ, int NWV, bool LX, bool MIX = false, int NTL = 4>
__global__ __launch_bounds__(NWV * 64) void k_qkv_mfma(LayerArgs A) {
  constexpr int BR = 16 * NTL;          // rows per block: NTL row tiles of 16
  constexpr int KW = KQ * 4 / NWV;      // 32-wide steps of this wave's share of the contraction
  // steps per operand batch (x of four row tiles); LX: 4 steps = 16 KB of x per wave
  constexpr int KC = LX ? 4 : (KW < 8 ? KW : 8);
  static_assert(!LX || (NWV == 8 && KW % 4 == 0), "x staging: 16 KB per wave and batch");
  extern __shared__ __align__(16) unsigned char dyn[];   // LX: [NWV][BR rows][256 B] x, then the wave's sums
  __shared__ f32x4_t s_cs[LX ? 1 : NWV][NTL][kWave];
  __shared__ float s_ss[NWV][BR];
  __shared__ float2 s_rope[BR][8];   // (cos, sin) for the block's rows x its 8 rotary pairs
  // the waves' sums: LX in each wave's own staging region (its x is read by then)
  auto s_c_at = [&](int wv, int nt) __attribute__((always_inline)) -> f32x4_t * {
    if constexpr (LX) return reinterpret_cast<f32x4_t *>(dyn + wv * 16384) + nt * kWave;
    else return &s_cs[wv][nt][0];
  };
  const int wave = wave_id(), lane = lane_id();
  const int rtiles = (A.rows + BR - 1) / BR;
  const TileMap tm = tile_of(blockIdx.x, rtiles);
  const int tile = tm.col, nb = tm.row * BR;
  const int head = tile / kTilesPerHead, jj = tile % kTilesPerHead, t0 = 8 * jj;
  const int i16 = lane % 16, g4 = lane / 16;
  const int arow = head * kHeadDim + (i16 < 8 ? t0 + i16 : 64 + t0 + i16 - 8);
  const int H = A.H;
  const int kq0 = wave * (H / NWV) + g4 * 8;     // this lane's first k
  const uint16_t *wp = A.w_qkv + (size_t)arow * H + kq0;
  const uint16_t *xr[NTL];
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) xr[nt] = A.x + (size_t)min(nb + nt * 16 + i16, A.rows - 1) * H + kq0;
  if (blockIdx.x == 0) write_row_table<false, MIX>(A);
  const bool rot = head < A.nq + A.nkv;
  const uint16_t *gp = head < A.nq ? A.g_q : A.g_k;
  // the q/k norm gains of this lane's four outputs, requested ahead of the operands
  float gq4[4] = {1.f, 1.f, 1.f, 1.f};
  if (rot) {
#pragma unroll
    for (int j = 0; j < 4; ++j) gq4[j] = cvt16<DT>(gp[t0 + (g4 & 1) * 4 + j + (g4 < 2 ? 0 : 64)]);
  }

  f32x4_t acc[NTL];
  float ss[NTL];
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) {
    acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    ss[nt] = 0.f;
  }
#pragma unroll 1
  for (int c0 = 0; c0 < KW; c0 += KC) {
    uint4 w[KC], g[KC], x[NTL][KC];
    uint4 xl[LX ? 4 * NTL : 1];
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      if constexpr (LX) {   // W too as whole lines: instruction s, rows 4 s .. 4 s + 3 of the tile
        const int f = s * 64 + lane, r = f >> 4, ch = f & 15;
        const int wrow = head * kHeadDim + (r < 8 ? t0 + r : 64 + t0 + r - 8);
        w[s] = ld16_stream(A.w_qkv + (size_t)wrow * H + wave * (H / NWV) + c0 * 32 + ch * 8);
      } else {
        w[s] = ld16_stream(wp + (c0 + s) * 32);
      }
      g[s] = ld16(A.g_in + kq0 + (c0 + s) * 32);
      if constexpr (!LX) {
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) x[nt][s] = ld16(xr[nt] + (c0 + s) * 32);
      }
    }
    if constexpr (LX) {   // instruction j: rows 4 j .. 4 j + 3, sixteen 16-byte chunks each
#pragma unroll
      for (int j = 0; j < 4 * NTL; ++j) {
        const int f = j * 64 + lane, r = f >> 4, ch = f & 15;
        xl[j] = ld16(A.x + (size_t)min(nb + r, A.rows - 1) * H + wave * (H / NWV) + c0 * 32 + ch * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch is issued before any math
    if (c0 == 0 && rot) {   // rotary angles of the block's rows x 8 pairs in fp64 while the operands travel
      for (int idx = threadIdx.x; idx < BR * 8; idx += NWV * 64) {
        const int r = idx / 8, tt = idx % 8;
        const int n = nb + r;
        float cs = 1.f, sn = 0.f;
        if (n < A.rows) {
          const double omega = exp2(-(2.0 * (t0 + tt) / kHeadDim) * log2((double)A.theta));
          double sd, cd;
          sincos((double)rope_pos<MIX>(A, n, t0 + tt) * omega, &sd, &cd);
          cs = (float)cd;
          sn = (float)sd;
        }
        s_rope[r][tt] = make_float2(cs, sn);
      }
    }
    if constexpr (LX) {   // own region, chunk ch of row r at chunk ch ^ (r & 15): both patterns conflict-free
      unsigned char *xw = dyn + wave * 16384;
      wave_lds_sync();   // the previous batch's reads of the region are done
#pragma unroll
      for (int j = 0; j < 4 * NTL; ++j) {
        const int f = j * 64 + lane, r = f >> 4, ch = f & 15;
        *reinterpret_cast<uint4 *>(xw + r * 256 + ((ch ^ (r & 15)) << 4)) = xl[j];
      }
      wave_lds_sync();   // x stored by every lane before any lane reads the operand layout
#pragma unroll
      for (int s = 0; s < KC; ++s)
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
          const int r = nt * 16 + i16, ch = s * 4 + g4;
          x[nt][s] = lds_ld16(reinterpret_cast<const uint16_t *>(xw + r * 256 + ((ch ^ (r & 15)) << 4)));
        }
      // then W's 16 rows x 256 B through the first 4 KB of the same region (its x is in registers now)
      wave_lds_sync();   // every lane's x reads done before W overwrites them
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        const int f = s * 64 + lane, r = f >> 4, ch = f & 15;
        *reinterpret_cast<uint4 *>(xw + r * 256 + ((ch ^ r) << 4)) = w[s];
      }
      wave_lds_sync();   // W stored before the operand-layout reads
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        const int ch = s * 4 + g4;
        w[s] = lds_ld16(reinterpret_cast<const uint16_t *>(xw + i16 * 256 + ((ch ^ i16) << 4)));
      }
    }
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      uint4 ahi, alo;
      {
        float wf[8], gf[8], p[8];
        unpack8<DT>(w[s], wf);
        unpack8<DT>(g[s], gf);
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = wf[e] * gf[e];
        split8<DT>(p, ahi, alo);
      }
#pragma unroll
      for (int nt = 0; nt < NTL; ++nt) {
        ss[nt] = sumsq8<DT>(x[nt][s], ss[nt]);   // the row sums of squares on the packed dot
        acc[nt] = mfma16x16x32<DT>(ahi, x[nt][s], acc[nt]);
        acc[nt] = mfma16x16x32<DT>(alo, x[nt][s], acc[nt]);
      }
    }
  }
  if constexpr (LX) wave_lds_sync();   // W reads done before the sums overwrite the region
#pragma unroll
  for (int nt = 0; nt < NTL; ++nt) {
    s_c_at(wave, nt)[lane] = acc[nt];
    float v = ss[nt];
    v = xsum<16>(v);
    v = xsum<32>(v);
    if (g4 == 0) s_ss[wave][nt * 16 + i16] = v;
  }
  __syncthreads();
  if (wave < NTL) {   // wave nt finishes row tile nt
    const int nt = wave;
    const int n = nb + nt * 16 + i16;
    f32x4_t c = s_c_at(0, nt)[lane];
    float ssx = s_ss[0][nt * 16 + i16];
#pragma unroll
    for (int wv = 1; wv < NWV; ++wv) {
      const f32x4_t d = s_c_at(wv, nt)[lane];
      c[0] += d[0]; c[1] += d[1]; c[2] += d[2]; c[3] += d[3];
      ssx += s_ss[wv][nt * 16 + i16];
    }
    const float inv = 1.0f / sqrtf(ssx / (float)H + A.eps);
    const bool first = g4 < 2;
    float raw[4], out[4];
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      raw[j] = c[j] * inv;
      sq += raw[j] * raw[j];
    }
    sq = xsum<16>(sq);
    sq = xsum<32>(sq);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tt = (g4 & 1) * 4 + j;
      if (rot) {
        const float u = gq4[j] * raw[j];
        const float up = xpartner32(u);
        const float2 cs = s_rope[nt * 16 + i16][tt];
        out[j] = first ? u * cs.x - up * cs.y : u * cs.x + up * cs.y;
      } else {
        out[j] = raw[j];
      }
    }
    if (n < A.rows) {
      const int t = t0 + (g4 & 1) * 4;   // four consecutive outputs: one 16-byte store
      *reinterpret_cast<float4 *>(A.qkv + (size_t)n * A.nqkv + head * kHeadDim + (first ? t : t + 64)) =
          make_float4(out[0], out[1], out[2], out[3]);
      if (rot && g4 == 0) A.ssq[((size_t)n * (A.nq + A.nkv) + head) * kTilesPerHead + jj] = sq;
    }
  }
}

// o_proj: out[n][o] = sum_c W_o[o][c] att[n][c] (+ residual), att as hi + lo terms
// read from its tiled copy [plane][c / 32][row][32].
// LW (nq d = 2048, eight waves): each wave loads its 16 W_o rows x 512 bytes
// as whole lines (two rows per instruction) into its own 8 KB of LDS and reads
// the operand layout back (chunk c of row r stored at chunk c ^ (r mod 16)).
template <int DT, int KQ, int NWV, bool LW, bool MIX = false>
__global__ __launch_bounds__(NWV * 64) void k_oproj_mfma(LayerArgs A) {
  constexpr int KW = KQ * 4 / NWV;   // 32-wide steps of this wave's share of the contraction
  constexpr int KC = chunk_steps(KW);
  static_assert(!LW || (KQ == 16 && NWV == 8 && KC == 8), "W staging: 8 KB per wave, one batch");
  extern __shared__ __align__(16) unsigned char dyn[];   // LW: [NWV][16 rows][512 B] of W_o
  __shared__ f32x4_t s_c[NWV][kWave];
  const int wave = wave_id(), lane = lane_id();
  const int i16 = lane % 16, g4 = lane / 16;
  const int K = A.nq * kHeadDim;
  const int rtiles = (A.rows + 15) / 16;
  const TileMap tm = tile_of(blockIdx.x, rtiles);
  const int o0 = tm.col * 16, nb = tm.row * 16;
  const int kq0 = wave * (K / NWV) + g4 * 8;
  const uint16_t *wp = A.w_o + (size_t)(o0 + i16) * K + kq0;
  const size_t plane = (size_t)(K / 32) * A.rows * 32;
  const size_t kstep = (size_t)A.rows * 32;   // next 32-wide block of the contraction
  const uint16_t *bp = A.att_hl + ((size_t)(wave * (K / (32 * NWV))) * A.rows + min(nb + i16, A.rows - 1)) * 32 + g4 * 8;
  // what the epilogue reads besides the products, requested first (wave 0 writes the tile)
  const int n_out = nb + i16;
  bool row_ok = false;
  float res4[4] = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0 && n_out < A.rows) {
    row_ok = A.rowtab[n_out].x != 0;
    if (A.residual) {
#pragma unroll
      for (int j = 0; j < 4; ++j) res4[j] = cvt16<DT>(A.residual[(size_t)n_out * A.H + o0 + g4 * 4 + j]);
    }
  }
  if (blockIdx.x == 0) advance_lengths<false, MIX>(A);

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int c0 = 0; c0 < KW; c0 += KC) {
    uint4 w[KC], hi[KC], lo[KC];
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      if constexpr (LW) {   // instruction s: rows 2 s, 2 s + 1, thirty-two 16-byte chunks each
        const int f = s * 64 + lane, r = f >> 5, ch = f & 31;
        w[s] = ld16_stream(A.w_o + (size_t)(o0 + r) * K + wave * (K / NWV) + ch * 8);
      } else {
        w[s] = ld16_stream(wp + (c0 + s) * 32);
      }
      hi[s] = ld16(bp + (c0 + s) * kstep);
      lo[s] = ld16(bp + plane + (c0 + s) * kstep);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the batch is issued before any math
    if constexpr (LW) {
      unsigned char *ww = dyn + wave * 8192;
      wave_lds_sync();   // the previous batch's reads of the region are done
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        const int f = s * 64 + lane, r = f >> 5, ch = f & 31;
        *reinterpret_cast<uint4 *>(ww + r * 512 + ((ch ^ (r & 15)) << 4)) = w[s];
      }
      wave_lds_sync();   // W_o stored by every lane before the operand-layout reads
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        const int ch = s * 4 + g4;
        w[s] = lds_ld16(reinterpret_cast<const uint16_t *>(ww + i16 * 512 + ((ch ^ i16) << 4)));
      }
    }
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      acc = mfma16x16x32<DT>(w[s], hi[s], acc);
      acc = mfma16x16x32<DT>(w[s], lo[s], acc);
    }
  }
  s_c[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const int n = nb + i16;
    f32x4_t c = s_c[0][lane];
#pragma unroll
    for (int wv = 1; wv < NWV; ++wv) {
      const f32x4_t d = s_c[wv][lane];
      c[0] += d[0]; c[1] += d[1]; c[2] += d[2]; c[3] += d[3];
    }
    if (n < A.rows) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t o = (size_t)n * A.H + o0 + g4 * 4 + j;
        float val = c[j];
        if (A.residual) val += res4[j];
        if (!row_ok) val = __builtin_nanf("");
        if (A.out_f32) reinterpret_cast<float *>(A.out)[o] = val;
        else reinterpret_cast<uint16_t *>(A.out)[o] = rne16<DT>(val);
      }
    }
  }
}

// dynamic LDS of phase C: the appended K/V rows of an item, then the item prefix
__host__ __device__ __forceinline__ size_t lds_attn_bytes(int rows, int n) {
  return (size_t)rows * sizeof(int4) + (size_t)n * kHeadDim * 2 * sizeof(uint16_t) + (size_t)(rows + 1) * sizeof(int);
}

template <int DT, int KV, int RB>
__global__ __launch_bounds__(256) void k_qkv(LayerArgs A) {
  __shared__ float s_ssq[RB][4];
  uint4 wr[4][KV];
  qkv_tile<DT, KV, RB, false, true>(A, blockIdx.x, s_ssq, wr);
  if (blockIdx.x == 0) write_row_table<false>(A);
  if (A.oproj_split) {   // the fp32 output that the two o_proj halves add into
    const int n4 = A.rows * A.H / 4;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += gridDim.x * blockDim.x)
      reinterpret_cast<float4 *>(A.out)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <int DT, int GROUP, bool MIX = false, bool PG = false>
__global__ __launch_bounds__(256) void k_attn(LayerArgs A) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ AttnShared<GROUP> S;
  int4 *rinfo = reinterpret_cast<int4 *>(dyn);
  uint16_t *knew = reinterpret_cast<uint16_t *>(rinfo + A.rows);
  uint16_t *vnew = knew + A.n * kHeadDim;
  int *pre = reinterpret_cast<int *>(vnew + A.n * kHeadDim);
  build_item_prefix<false, MIX>(A, pre, rinfo, S.wsum);
  attention_phase<DT, GROUP, false, PG>(A, pre, rinfo, knew, vnew, S, blockIdx.x, gridDim.x);
}

// ---------------------------------------------------------------- phase C for a few rows
//
// With a few rows (bs1 decode, short verify) the attention is a chain of
// latencies, not a stream, so nothing in it waits for another workgroup.
// Workgroup (row, g, c0) of a grid sized from the host's view of the lengths
// (A.nch_host chunks per row) takes chunk c0 of (row, g), and every
// nch_host-th after it should the device lengths exceed that view.  NW waves
// share a chunk: wave w takes keys t0 + 8 (NW i + w) + (0..7) at step i, one
// key row per group of 8 lanes.  The first NP steps of every wave, its q heads
// and the appended rows it may see are requested at once, before the row's
// length is known: the K/V rows are clamped into the cache, so the loads are in
// bounds for any length, and keys found to be past the visible ones are
// masked.  Wave w < n holds the sequence's appended row w (n <= 4 here).
// Softmax over the loaded steps as one block: all scores, one maximum per
// head, then the weights (steps past NP, if any, continue online).  The waves'
// sums are reduce-scattered over their key groups, combined in LDS, and the
// partial (m, l, acc) is the output; the o_proj kernel merges the partials of
// a row as it reads them (k_oproj_merge).
template <int NW, int GROUP>
struct FewShared {
  float acc[NW][GROUP][kHeadDim];
  float m[NW][GROUP], l[NW][GROUP];
};

struct FewGeom {
  int L, t0, t1, nb, n_new, tw, nsteps, last_row;
  size_t kvrow0;
  int slot, g;
};

template <int NW>
__device__ __forceinline__ FewGeom few_geom(const LayerArgs &A, int slot, int g, int L, int nvis, int c) {
  FewGeom G;
  G.L = L;
  G.t0 = c * A.split;
  G.t1 = min(G.t0 + A.split, nvis);
  G.nb = max(G.t0, L);
  G.n_new = max(0, G.t1 - G.nb);
  G.kvrow0 = ((size_t)slot * A.nkv + g) * A.capacity;
  G.slot = slot;
  G.g = g;
  G.tw = G.t0 + wave_id() * 8;
  G.nsteps = G.tw < G.t1 ? (G.t1 - G.tw + NW * 8 - 1) / (NW * 8) : 0;
  G.last_row = max(min(G.t1, L) - 1, 0);
  return G;
}

// PG (paged cache): a step's rows, 8-aligned and clamped to the chunk's last
// committed row, lie in one page (a page holds at least 16 rows), whose id is a
// wave-uniform value; an id outside the pool (possible for rows requested
// before the length is known, which are then never used) reads page 0.
template <int NW, bool PG = false>
__device__ __forceinline__ void few_load_step(const LayerArgs &A, const FewGeom &G, uint4 (&r)[4], int i) {
  const int lane = lane_id(), kl = lane & 7, kr = lane >> 3;
  if constexpr (PG) {
    const int t = G.tw + NW * 8 * i;
    const int pid = page_entry(A, G.slot, min(t, G.last_row) >> A.plog);
    const int page = (unsigned)pid < (unsigned)A.npages ? pid : 0;
    const int row = min(t + kr, G.last_row);
    const size_t e = (((size_t)page * A.nkv + G.g) * A.psz + (row & (A.psz - 1))) * kHeadDim + kl * 8;
    r[0] = ld16(A.kc + e);
    r[1] = ld16(A.kc + e + 64);
    r[2] = ld16(A.vc + e);
    r[3] = ld16(A.vc + e + 64);
    return;
  }
  const uint32_t region = (uint32_t)A.capacity * kHeadDim * 2;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(A.kc + G.kvrow0 * kHeadDim, region);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(A.vc + G.kvrow0 * kHeadDim, region);
  const uint32_t off = (uint32_t)min(G.tw + NW * 8 * i + kr, G.last_row) * (kHeadDim * 2) + kl * 16;
  r[0] = ld_buf(Kr, off);
  r[1] = ld_buf(Kr, off + 128);
  r[2] = ld_buf(Vr, off);
  r[3] = ld_buf(Vr, off + 128);
}

template <int DT, int GROUP, int NW, int NP, bool PG = false>
__device__ __forceinline__ void few_stream(const LayerArgs &A, const FewGeom &G, int row, int g, int c,
                                           const float (&q)[GROUP][16], const uint16_t *knew, const uint16_t *vnew,
                                           FewShared<NW, GROUP> &S, uint4 (&r)[NP][4]) {
  static_assert(NP >= 2, "two register sets at least");
  const int wave = wave_id(), lane = lane_id();
  const int kl = lane & 7, kr = lane >> 3;
  const int d0 = 8 * kl, d1 = 64 + 8 * kl;
  const int nsteps = G.nsteps;
  // K (h = 0) or V (h = 1) of step i as the cache holds it: appended keys from LDS, keys past the chunk zero
  auto operand = [&](const uint4 (&rr)[4], int i, int h, bool with_new, uint4 &x0, uint4 &x1) __attribute__((always_inline)) {
    const int t = G.tw + NW * 8 * i + kr;
    const bool valid = t < G.t1;
    x0 = rr[2 * h];
    x1 = rr[2 * h + 1];
    if (with_new) {
      const bool fresh = valid && t >= G.L;
      const uint16_t *src = (h == 0 ? knew : vnew) + (fresh ? t - G.nb : 0) * kHeadDim;
      const uint4 a0 = lds_ld16(src + d0), a1 = lds_ld16(src + d1);
      if (fresh) {
        x0 = a0;
        x1 = a1;
      }
    }
    // V rows past the chunk are zeroed (their weight is 0, but 0 * inf is not);
    // K rows need not be: their scores are replaced by -inf.  A step whose
    // keys are all visible (wave-uniform) skips the masking.
    if (h == 1 && G.tw + NW * 8 * i + 7 >= G.t1) {
      const uint32_t vm = valid ? 0xffffffffu : 0u;
      x0 = make_uint4(x0.x & vm, x0.y & vm, x0.z & vm, x0.w & vm);
      x1 = make_uint4(x1.x & vm, x1.y & vm, x1.z & vm, x1.w & vm);
    }
    return valid;
  };
  auto score = [&](const uint4 (&rr)[4], int i, bool with_new, float (&s)[GROUP]) __attribute__((always_inline)) {
    uint4 k0, k1;
    const bool valid = operand(rr, i, 0, with_new, k0, k1);
    float kf[16];
    unpack8<DT>(k0, kf);
    unpack8<DT>(k1, kf + 8);
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      float xp[4] = {0.f, 0.f, 0.f, 0.f};   // four independent chains
#pragma unroll
      for (int e = 0; e < 16; ++e) xp[e & 3] += q[j][e] * kf[e];
      const float x = sum8((xp[0] + xp[1]) + (xp[2] + xp[3]));
      s[j] = valid ? x : -INFINITY;
    }
  };
  float m[GROUP], l[GROUP], acc[GROUP][16];
  auto weigh = [&](const uint4 (&rr)[4], int i, bool with_new, const float (&s)[GROUP]) __attribute__((always_inline)) {
    uint4 v0, v1;
    operand(rr, i, 1, with_new, v0, v1);
    float vf[16];
    unpack8<DT>(v0, vf);
    unpack8<DT>(v1, vf + 8);
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      const float p = s[j] == -INFINITY ? 0.f : exp2_neg(s[j] - m[j]);
      l[j] += p;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] += p * vf[e];
    }
  };
  auto run = [&](bool with_new) __attribute__((always_inline)) {
    // the NP loaded steps as one block
    float sc[NP][GROUP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      if (k < nsteps) score(r[k], k, with_new, sc[k]);
      else
#pragma unroll
        for (int j = 0; j < GROUP; ++j) sc[k][j] = -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < GROUP; ++j) {
      float x = sc[0][j];
#pragma unroll
      for (int k = 1; k < NP; ++k) x = fmaxf(x, sc[k][j]);
      x = fmaxf(x, dpp<kRowMirror>(x));   // the two key groups of a 16-lane row, then the four rows
      m[j] = fmaxf(fmaxf(readlane(x, 0), readlane(x, 16)), fmaxf(readlane(x, 32), readlane(x, 48)));
      l[j] = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < NP; ++k)
      if (k < nsteps) weigh(r[k], k, with_new, sc[k]);
    // further steps (device lengths beyond the host's view): online, two in flight
    if (nsteps > NP) {
      uint4 (&ra)[4] = r[0];
      uint4 (&rb)[4] = r[NP - 1];
      few_load_step<NW, PG>(A, G, ra, NP);
      few_load_step<NW, PG>(A, G, rb, NP + 1);
      auto online = [&](const uint4 (&rr)[4], int i) __attribute__((always_inline)) {
        float s[GROUP];
        score(rr, i, with_new, s);
#pragma unroll
        for (int j = 0; j < GROUP; ++j) {
          float x = fmaxf(s[j], dpp<kRowMirror>(s[j]));
          x = fmaxf(fmaxf(readlane(x, 0), readlane(x, 16)), fmaxf(readlane(x, 32), readlane(x, 48)));
          if (x > m[j]) {   // wave-uniform
            const float corr = exp2_neg(m[j] - x);   // 0 while m = -inf
            m[j] = x;
            l[j] *= corr;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] *= corr;
          }
        }
        weigh(rr, i, with_new, s);
      };
      int i = NP;
      for (; i + 2 < nsteps; i += 2) {
        online(ra, i);
        few_load_step<NW, PG>(A, G, ra, i + 2);
        online(rb, i + 1);
        few_load_step<NW, PG>(A, G, rb, i + 3);
      }
      if (i < nsteps) online(ra, i);
      if (i + 1 < nsteps) online(rb, i + 1);
    }
  };
  if (G.n_new == 0) run(false);
  else run(true);

  // sum over the wave's 8 key groups: reduce-scatter over lane bits 5, 4, 3
  constexpr int N = GROUP * 16;
  float v1[N], v2[N / 2], v3[N / 4], v4[N / 8];
#pragma unroll
  for (int j = 0; j < GROUP; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) v1[j * 16 + e] = acc[j][e];
  rs_half<N, 32>(v1, v2);
  rs_half<N / 2, 16>(v2, v3);
  rs_half<N / 4, 8>(v3, v4);
  const int base = ((lane >> 5) & 1) * (N / 2) + ((lane >> 4) & 1) * (N / 4) + ((lane >> 3) & 1) * (N / 8);
#pragma unroll
  for (int u = 0; u < N / 8; ++u) {
    const int i = base + u, j = i / 16, e = i % 16;
    S.acc[wave][j][e < 8 ? d0 + e : d1 + e - 8] = v4[u];
  }
#pragma unroll
  for (int j = 0; j < GROUP; ++j) {
    float x = l[j];
    x = xsum<32>(x);
    x = xsum<16>(x);
    x = xsum<8>(x);
    if (lane == 0) {
      S.m[wave][j] = m[j];
      S.l[wave][j] = x;
    }
  }
  __syncthreads();
  float *pbase = A.part + ((((size_t)row * A.nkv + g) * kMaxChunks + c) * GROUP) * kPartStride;
  for (int idx = threadIdx.x; idx < GROUP * kHeadDim; idx += NW * kWave) {
    const int j = idx / kHeadDim, d = idx % kHeadDim;
    float M = S.m[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, S.m[w][j]);
    float a = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = S.m[w][j] == -INFINITY ? 0.f : exp2_neg(S.m[w][j] - M);
      a += sc * S.acc[w][j][d];
      ls += sc * S.l[w][j];
    }
    pbase[j * kPartStride + d] = a;
    if (d == 0) {
      pbase[j * kPartStride + 128] = M;
      pbase[j * kPartStride + 129] = ls;
    }
  }
  __syncthreads();
}

template <int DT, int GROUP, int NW, int NP, bool PG = false>
__global__ __launch_bounds__(NW * 64) void k_attn_few(LayerArgs A) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ FewShared<NW, GROUP> S;
  uint16_t *knew = reinterpret_cast<uint16_t *>(dyn);
  uint16_t *vnew = knew + A.n * kHeadDim;
  const int C = A.nch_host;
  const int row = blockIdx.x / (A.nkv * C), g = (blockIdx.x / C) % A.nkv, c0 = blockIdx.x % C;
  const int wave = wave_id(), lane = lane_id();
  const int b = seq_of(A, row), r_off = row - seq_row0(A, b);
  // the slot as far as the loads need it: a sequence's own without a slot
  // table, else its entry clamped into the cache (rows of a bad slot are masked)
  const int slot = A.slots ? min(max(A.slots[b], 0), A.batch_cap - 1) : b;
  FewGeom G0 = few_geom<NW>(A, slot, g, A.capacity, A.capacity, c0);
  G0.last_row = A.capacity - 1;
  uint4 rr[NP][4];
#pragma unroll
  for (int k = 0; k < NP; ++k) few_load_step<NW, PG>(A, G0, rr[k], k);
  QLoads<GROUP> Q;
  q_loads<GROUP>(A, row, g, Q);
  const bool has_fresh = wave <= r_off;   // sequence row `wave`, position L + wave, is visible to `row`
  float4 fk = make_float4(0.f, 0.f, 0.f, 0.f), fv = fk, fp0 = fk, fp1 = fk;
  if (has_fresh) {
    const int rrow = row - r_off + wave;
    const __amdgpu_buffer_rsrc_t Rr = rsrc_of(A.qkv + (size_t)rrow * A.nqkv, (uint32_t)A.nqkv * 4);
    fk = ld_dev4(Rr, ((A.nq + g) * kHeadDim + 2 * (lane & ~1)) * 4);
    fv = ld_dev4(Rr, ((A.nq + A.nkv + g) * kHeadDim + 2 * (lane & ~1)) * 4);
    const __amdgpu_buffer_rsrc_t Pr = rsrc_of(A.ssq + (size_t)rrow * (A.nq + A.nkv) * kTilesPerHead,
                                              (uint32_t)(A.nq + A.nkv) * kTilesPerHead * 4);
    fp0 = ld_dev4(Pr, (A.nq + g) * kTilesPerHead * 4);
    fp1 = ld_dev4(Pr, ((A.nq + g) * kTilesPerHead + 4) * 4);
  }
  const RowInfo ri = row_info(A, row);
  const int nch = chunks_of(ri.nvis, A.split);   // 0 for a row in error
  if (c0 >= nch) return;                          // uniform over the workgroup
  float q[GROUP][16];
  q_scale<GROUP>(A, Q, q);
  for (int c = c0; c < nch; c += C) {
    const FewGeom G = few_geom<NW>(A, ri.slot, g, ri.L, ri.nvis, c);
    if (c != c0) {
#pragma unroll
      for (int k = 0; k < NP; ++k) few_load_step<NW, PG>(A, G, rr[k], k);
    }
    if (G.n_new > 0) {
      const int i = ri.L + wave - G.nb;   // this wave's row among the chunk's appended ones
      if (has_fresh && i >= 0 && i < G.n_new) {
        uint32_t kb, vb;
        fresh_pair<DT>(A, fk, fv, fp0, fp1, kb, vb);
        reinterpret_cast<uint32_t *>(knew + i * kHeadDim)[lane] = kb;
        reinterpret_cast<uint32_t *>(vnew + i * kHeadDim)[lane] = vb;
        if (wave == r_off) {   // every row also stores its own appended row in the cache
          size_t off = (G.kvrow0 + ri.L + wave) * kHeadDim;
          bool store = true;
          if constexpr (PG) {   // row (L + wave) % psz of its page; not stored for an id outside the pool
            const int t = ri.L + wave;
            const int pid = page_entry(A, ri.slot, t >> A.plog);
            store = (unsigned)pid < (unsigned)A.npages;
            off = (((size_t)(store ? pid : 0) * A.nkv + g) * A.psz + (t & (A.psz - 1))) * kHeadDim;
          }
          if (store) {
            reinterpret_cast<uint32_t *>(A.kc + off)[lane] = kb;
            reinterpret_cast<uint32_t *>(A.vc + off)[lane] = vb;
          }
        }
      }
      __syncthreads();
    }
    few_stream<DT, GROUP, NW, NP, PG>(A, G, row, g, c, q, knew, vnew, S, rr);
    if constexpr (PG) {
      // the chunk's pages, now that its keys are known: an id outside the pool is reported
      if (wave == 0) {
        const int p0 = G.t0 >> A.plog, npg = ((G.t1 - 1) >> A.plog) - p0 + 1;
        const int pid = A.ptab[(size_t)ri.slot * A.pps + min(p0 + lane, A.pps - 1)];
        if (__any(lane < npg && (unsigned)pid >= (unsigned)A.npages) && lane == 0 && A.status)
          atomicOr(A.status, kStatusBadPage);
      }
    }
  }
}

// many rows: equal key shares per wave of a resident grid
template <int DT, int GROUP, bool NT, bool F8, bool MIX = false, bool PG = false>
__global__ __launch_bounds__(256) void k_attn_waves(LayerArgs A) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ int wsum[4];
  int4 *rinfo = reinterpret_cast<int4 *>(dyn);
  int *pre = reinterpret_cast<int *>(rinfo + A.rows);
  build_item_prefix<true, MIX>(A, pre, rinfo, wsum);
  attention_waves<DT, GROUP, NT, F8, PG>(A, pre, rinfo, blockIdx.x * 4 + wave_id(), gridDim.x * 4);
}

__host__ __device__ __forceinline__ size_t lds_attn_waves_bytes(int rows) {
  return (size_t)rows * sizeof(int4) + (size_t)(rows + 1) * sizeof(int);
}

// ---------------------------------------------------------------- phase C for verify blocks on the matrix cores
//
// The k rows of a verify block all read their sequence's cache, so here one
// work item streams each (sequence, kv head g, chunk of keys) once for a
// 16-row tile of the M = GROUP * k query rows of g (query row m = r * GROUP + h:
// block row r, q head g * GROUP + h); with 32 query rows the two tiles are two
// items of the same chunk (the second stream mostly hits the caches), which
// keeps one tile's operands per wave and leaves room for two K/V register sets.
// Per 32-key step of a wave:
//   S^T = K Q^T    v_mfma_f32_16x16x32, A = 16 keys x 32 dims of K (exact
//                  16-bit), B = the same dims of Q (two 16-bit terms, hi + lo)
//   O^T += V^T P^T A = 16 dims x 32 keys of V, B = the weights P (hi + lo)
// A lane of the score tile holds 4 keys of one query row, which is exactly its
// share of the B operand of the next product (the 32 keys are contracted in
// the order {4j..4j+3, 16+4j..16+4j+3} for lane group j, and V is read in the
// same order), so the weights never leave the registers.  K and V of a step
// arrive as whole 128-byte lines (four keys per load instruction) and pass
// through the wave's LDS region: K rows with chunk c at c ^ (key & 15) for the
// A-operand reads, V rows with chunk c at c ^ 2 (key & 7) for the transposing
// reads (ds_read_b64_tr_b16: lane p of each 16-lane group receives element
// p % 4 of the lanes 4 e + p / 4, e = 0..3, i.e. four keys of one dim).
// Online softmax per query row in base 2 (Q carries log2(e) / sqrt(d)); the
// four waves of an item combine in LDS into one partial per (row, q head) in
// the split-KV layout; the last item of a (sequence, g) to be counted merges
// the partials of all its rows in chunk order (deterministic).  Keys at or past
// the committed length are this call's rows, taken from the projection (k
// normalised, both rounded to 16 bits as stored) and written to the cache by
// the one step that holds them.

constexpr int kVmWaves = 4;    // waves per workgroup
constexpr int kVmStep = 32;    // keys per wave step
constexpr int kVmStage = 8192; // LDS bytes of one 32-key K (or V) stage
constexpr int kVmRow = 132;    // floats per query row of the combine buffer (padded against bank conflicts)

// dynamic LDS: per wave a K and a V stage (reused by the combine), then the
// sequences' item prefix and (slot, L, nvis, ok)
__host__ __device__ __forceinline__ size_t lds_vmfma_bytes(int B) {
  return (size_t)kVmWaves * 2 * kVmStage + (size_t)B * sizeof(int4) + (size_t)(B + 1) * sizeof(int);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_ld8_tr16(const unsigned char *p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t *)((__attribute__((address_space(3))) unsigned char *)p));
  return __builtin_bit_cast(uint2, r);
}

// block-wide exclusive prefix of the items (chunks x kv heads) of every sequence
__device__ void build_seq_prefix(const LayerArgs &A, int *pre, int4 *sinfo, int *wsum) {
  const int wave = wave_id(), lane = lane_id();
  const int B = A.B;
  const int per = (B + 255) / 256;
  const int beg = min((int)threadIdx.x * per, B), end = min(beg + per, B);
  int local = 0;
  for (int b = beg; b < end; ++b) {
    const RowInfo ri = row_info(A, seq_row0(A, b));
    const int nvis = ri.ok ? ri.L + seq_rows(A, b) : 0;
    sinfo[b] = make_int4(ri.slot, ri.L, nvis, (int)ri.ok);
    local += chunks_of(nvis, A.split) * A.nkv * A.vm_nt;
  }
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
  for (int b = beg; b < end; ++b) {
    pre[b] = run;
    run += chunks_of(sinfo[b].z, A.split) * A.nkv * A.vm_nt;
  }
  if (threadIdx.x == 255) pre[B] = run;
  __syncthreads();
}

// Merge of the np chunk partials of every (row r < k, head h) of one
// (sequence, kv head g) by the whole workgroup at once: the (m, l) of all
// chunks into LDS, one thread per (r, h) turns them into weights
// 2^(m_c - M) / sum_c 2^(m_c - M) l_c, then every thread sums float4 columns
// over the chunks in chunk order (deterministic) and writes the attention
// output and its hi / lo tiles.  `ws` is LDS scratch of 2 * k * GROUP * np floats.
// Merge of the np chunk partials of every (row r < k, head h) of one
// (sequence, kv head g) by the whole workgroup at once, in one memory round
// trip: every (m, l) and the first eight chunks of every output column are
// requested together.  Wave w turns the (m, l) of the pairs rh = w, w + 4, ...
// (rh = r * GROUP + h; lane c holds chunk c) into the weights
// 2^(m_c - M) / sum_c 2^(m_c - M) l_c by wave reductions and leaves them in
// LDS; then every thread sums its float4 columns over the chunks in chunk
// order (deterministic) and writes the attention output and its hi / lo
// tiles.  `ws`: LDS scratch of 32 * 64 floats; k * GROUP <= 32, np <= 64.
template <int DT, int GROUP>
__device__ void merge_block_vm(const LayerArgs &A, int row0, int k, int g, int np, float *ws) {
  constexpr int CPT = 4, BATCH = 8, PPW = 32 / kVmWaves;   // columns per thread, chunks per load batch, pairs per wave
  const int pairs = k * GROUP;
  const int wave = wave_id(), lane = lane_id();
  const uint32_t pstride = (uint32_t)kMaxChunks * GROUP * kPartStride;   // floats per (row, kv head)
  // one workgroup-uniform resource over the block's partials; per-lane offsets
  const __amdgpu_buffer_rsrc_t R =
      rsrc_of(A.part + ((size_t)row0 * A.nkv + g) * pstride, (uint32_t)((k - 1) * A.nkv + 1) * pstride * 4);
  auto at = [&](int rh, int c) -> uint32_t {   // byte offset of the partial of pair rh, chunk c
    return ((uint32_t)(rh / GROUP) * A.nkv * pstride + ((uint32_t)c * GROUP + rh % GROUP) * kPartStride) * 4;
  };
  float4 ml[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) ml[i] = ld_dev4(R, at(min(wave + kVmWaves * i, pairs - 1), min(lane, np - 1)) + 128 * 4);
  float4 v[CPT][BATCH];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int f = min((int)threadIdx.x + q * (int)blockDim.x, pairs * 32 - 1), rh = f / 32, d = (f % 32) * 4;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) v[q][u] = ld_dev4(R, at(rh, min(u, np - 1)) + d * 4);
  }
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int rh = wave + kVmWaves * i;
    if (rh < pairs) {
      const float m = lane < np ? ml[i].x : -INFINITY;
      const float M = wave_max(m);
      const float w = (lane < np && m != -INFINITY) ? exp2_neg(m - M) : 0.f;
      const float tot = wave_sum(w * ml[i].y);
      ws[rh * kWave + lane] = w / tot;
    }
  }
  __syncthreads();
  const size_t plane = (size_t)(A.nq * kHeadDim / 32) * A.rows * 32;
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int f = threadIdx.x + q * blockDim.x;
    if (f >= pairs * 32) break;
    const int rh = f / 32, d = (f % 32) * 4, r = rh / GROUP, h = rh % GROUP;
    const float *wv = ws + rh * kWave;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c0 = 0; c0 < np; c0 += BATCH) {
      if (c0 > 0) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) v[q][u] = ld_dev4(R, at(rh, min(c0 + u, np - 1)) + d * 4);
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const float w = c0 + u < np ? wv[c0 + u] : 0.f;
        a.x += w * v[q][u].x;
        a.y += w * v[q][u].y;
        a.z += w * v[q][u].z;
        a.w += w * v[q][u].w;
      }
    }
    const int row = row0 + r;
    const size_t col = (size_t)(g * GROUP + h) * kHeadDim + d;
    *reinterpret_cast<float4 *>(A.att + (size_t)row * A.nq * kHeadDim + col) = a;
    uint16_t hv[4], lv[4];
    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hv[e] = rne16<DT>(av[e]);
      lv[e] = rne16<DT>(av[e] - cvt16<DT>(hv[e]));
    }
    // tiled [plane][col / 32][row][32] for the MFMA o_proj: the four values are adjacent
    const size_t idx = ((col / 32) * A.rows + row) * 32 + col % 32;
    *reinterpret_cast<uint2 *>(A.att_hl + idx) =
        make_uint2((uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16));
    *reinterpret_cast<uint2 *>(A.att_hl + plane + idx) =
        make_uint2((uint32_t)lv[0] | ((uint32_t)lv[1] << 16), (uint32_t)lv[2] | ((uint32_t)lv[3] << 16));
  }
}

template <int DT, int GROUP, int QT, bool DB, int NT>
__global__ __launch_bounds__(kVmWaves * 64) void k_attn_vmfma(LayerArgs A) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ int wsum[4];
  __shared__ float s_ml[kVmWaves][2][16];   // a wave's (m, l) per query row of the tile being combined
  __shared__ uint32_t s_old;
  const bool hostmap = A.vm_items > 0;   // items laid out by the host from its copy of the lengths
  int4 *sinfo = reinterpret_cast<int4 *>(dyn + kVmWaves * 2 * kVmStage);
  int *pre = reinterpret_cast<int *>(sinfo + A.B);
  if (!hostmap) build_seq_prefix(A, pre, sinfo, wsum);
  const int total = hostmap ? A.vm_items : pre[A.B];
  const int wave = wave_id(), lane = lane_id();
  const int n16 = lane & 15, j4 = lane >> 4;
  unsigned char *stk = dyn + wave * 2 * kVmStage, *stv = stk + kVmStage;
  const float qs = kLog2e * rsqrtf((float)kHeadDim);
  const int k = A.n;
  const uint32_t row_bytes = (uint32_t)A.nqkv * 4;
  const uint32_t ssq_bytes = (uint32_t)(A.nq + A.nkv) * kTilesPerHead * 4;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // (sequence b, kv head g, first chunk) of the item; with the host's layout the
    // item of a sequence's last host chunk also takes the chunks past the host's view
    const int *ip = hostmap ? A.vm_pre : pre;
    int lo = 0, hi = A.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (ip[mid] <= item) lo = mid; else hi = mid;
    }
    // the item's indices are uniform over the workgroup: readfirstlane keeps them, and
    // the buffer resources built from them, in scalar registers (a resource the
    // compiler cannot prove uniform costs a loop around every load)
    const int b = rfl(lo), row0 = b * k;
    constexpr int nt = NT;   // query tiles (A.vm_nt): items (g, chunk, tile) of sequence b
    const int nch_i = rfl((ip[b + 1] - ip[b]) / (A.nkv * nt));   // chunks per kv head in the item layout
    const int rem = item - rfl(ip[b]);
    const int g = rem / (nch_i * nt), rc = rem - g * (nch_i * nt);
    const int c_first = rc / nt, m0 = (rc - c_first * nt) * 16 * QT;   // first query row of the item's tiles
    int slot, L, nvis;
    if (hostmap) {
      slot = rfl(A.slots ? A.slots[b] : b);
    } else {
      const int4 si = sinfo[b];
      slot = rfl(si.x);
      L = rfl(si.y);
      nvis = rfl(si.z);
    }
    // a slot outside the cache reads slot 0's lines (its rows are skipped below)
    const int lslot = (slot >= 0 && slot < A.batch_cap) ? slot : 0;
    const size_t kvbase = ((size_t)lslot * A.nkv + g) * A.capacity * kHeadDim;
    const __amdgpu_buffer_rsrc_t Kr = make_rsrc(A.kc + kvbase, (uint32_t)A.capacity * kHeadDim * 2);
    const __amdgpu_buffer_rsrc_t Vr = make_rsrc(A.vc + kvbase, (uint32_t)A.capacity * kHeadDim * 2);

    // DB (chunks of several steps per wave, one query tile): two register sets of
    // K/V lines, a wave's steps alternate between them, and the loads of step j + 2
    // are requested as soon as step j is in LDS, so two steps are in flight while
    // one is computed.  Every DB request is unconditional (rows clamped into the
    // chunk, so a request past the chunk re-reads its last row): the number of
    // loads behind each set is then fixed and a wait for one set never waits for
    // the other.  (With two query tiles the second set would not fit the register
    // file beside their operands.)
    static_assert(!DB || QT == 1, "two register sets beside one query tile");
    uint4 lk0[8], lv0[8], lk1[8], lv1[8];
    int tclamp = 0;   // loads stay at or below this key (lines the item fetches anyway)
    auto issue = [&](uint4 (&lk)[8], uint4 (&lv)[8], int ts) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = min(ts + 4 * i + j4, tclamp);
        const uint32_t off = (uint32_t)t * (kHeadDim * 2) + n16 * 16;
        lk[i] = ld_buf(Kr, off);
        lv[i] = ld_buf(Vr, off);
      }
    };
    constexpr int kRound = kVmWaves * kVmStep;   // keys of one step of all four waves
    // the wave's first two steps of the first chunk, requested before the length arrives
    // (with the host layout): rows clamped into the chunk and the cache
    tclamp = min(c_first * A.split + A.split, A.capacity) - 1;
    if (hostmap || c_first * A.split + wave * kVmStep < nvis) {
      issue(lk0, lv0, c_first * A.split + wave * kVmStep);
      if (DB) issue(lk1, lv1, c_first * A.split + wave * kVmStep + kRound);
    }
    // Q of the tile rows, requested with the K/V lines and before the length (a wait
    // on a vector load waits on every load issued before it)
    float4 qv[QT][4][2], qp[QT][2];
    {
      const __amdgpu_buffer_rsrc_t Qr = make_rsrc(A.qkv + (size_t)row0 * A.nqkv, (uint32_t)k * row_bytes);
      const __amdgpu_buffer_rsrc_t Sr =
          make_rsrc(A.ssq + (size_t)row0 * (A.nq + A.nkv) * kTilesPerHead, (uint32_t)k * ssq_bytes);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int m = m0 + qt * 16 + n16, r = m / GROUP, h = m % GROUP;
        const uint32_t rr = (uint32_t)min(r, k - 1);   // rows past the block: zero weight below
        const uint32_t head = (uint32_t)(g * GROUP + h);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t o = rr * row_bytes + (head * kHeadDim + 32 * s + 8 * j4) * 4;
          qv[qt][s][0] = __builtin_bit_cast(float4, ld_buf(Qr, o));
          qv[qt][s][1] = __builtin_bit_cast(float4, ld_buf(Qr, o + 16));
        }
        qp[qt][0] = __builtin_bit_cast(float4, ld_buf(Sr, rr * ssq_bytes + head * kTilesPerHead * 4));
        qp[qt][1] = __builtin_bit_cast(float4, ld_buf(Sr, rr * ssq_bytes + head * kTilesPerHead * 4 + 16));
      }
    }
    if (hostmap) {
      const RowInfo ri = row_info(A, row0);
      L = rfl(ri.L);
      nvis = rfl(ri.ok ? ri.L + k : 0);
    }
    const int nch = chunks_of(nvis, A.split);
    const int c_last = (hostmap && c_first == nch_i - 1) ? max(nch, nch_i) - 1 : c_first;

    // Q as B operands: lane (query row n16 of tile qt, dims 32 s + 8 j4 .. + 7), two 16-bit terms
    uint4 qh[QT][4], ql[QT][4];
    {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int m = m0 + qt * 16 + n16;
        const float sc = (m / GROUP < k) ? inv_rms_of(A, qp[qt][0], qp[qt][1]) * qs : 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float f[8] = {qv[qt][s][0].x * sc, qv[qt][s][0].y * sc, qv[qt][s][0].z * sc, qv[qt][s][0].w * sc,
                              qv[qt][s][1].x * sc, qv[qt][s][1].y * sc, qv[qt][s][1].z * sc, qv[qt][s][1].w * sc};
          split8<DT>(f, qh[qt][s], ql[qt][s]);
        }
      }
    }

    for (int c = c_first; c <= c_last; ++c) {
    if (c >= nch) break;   // past the sequence's visible keys (the length shrank since the launch)
    const int cbeg = c * A.split, cend = min(cbeg + A.split, nvis);
    int t0 = cbeg + wave * kVmStep;
    tclamp = max(min(cend, L) - 1, 0);
    if (c > c_first && t0 < cend) {
      issue(lk0, lv0, t0);
      if (DB) issue(lk1, lv1, t0 + kRound);
    }
    float mrun[QT], lrun[QT];
    f32x4_t o[QT][8];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      mrun[qt] = -INFINITY;
      lrun[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[qt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // one step: set (lk, lv) holds keys [t0, t0 + 32) of this wave
    auto vstep = [&](uint4 (&lk)[8], uint4 (&lv)[8]) __attribute__((always_inline)) {
      wave_lds_sync();   // the previous step's operand reads are done
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kl = 4 * i + j4;
        *reinterpret_cast<uint4 *>(stk + kl * 256 + ((n16 ^ (kl & 15)) << 4)) = lk[i];
        *reinterpret_cast<uint4 *>(stv + kl * 256 + ((n16 ^ ((kl & 7) << 1)) << 4)) = lv[i];
      }
      if (t0 + kVmStep > L || t0 + kVmStep > cend) {
        // this call's rows (keys L .. L + k - 1) replace what was loaded for them: taken from the
        // projection as the cache stores them (k normalised, both rounded) and written to the
        // cache here, by the one step that holds them; keys past the chunk become zeros
        wave_lds_sync();
        const __amdgpu_buffer_rsrc_t Rr = make_rsrc(A.qkv + (size_t)row0 * A.nqkv, (uint32_t)k * row_bytes);
        const __amdgpu_buffer_rsrc_t Pr =
            make_rsrc(A.ssq + (size_t)row0 * (A.nq + A.nkv) * kTilesPerHead, (uint32_t)k * ssq_bytes);
#pragma unroll 1
        for (int pc = lane; pc < kVmStep * 16; pc += kWave) {
          const int kl = pc >> 4, ch = pc & 15, t = t0 + kl;
          if (t < L) continue;
          uint4 kq = make_uint4(0u, 0u, 0u, 0u), vq = kq;
          if (t < cend) {
            const uint32_t rr = (uint32_t)(t - L);
            const uint32_t kh = rr * row_bytes + ((A.nq + g) * kHeadDim + 8 * ch) * 4;
            const uint32_t vh = rr * row_bytes + ((A.nq + A.nkv + g) * kHeadDim + 8 * ch) * 4;
            const uint32_t ph = rr * ssq_bytes + (A.nq + g) * kTilesPerHead * 4;
            const float4 ka = __builtin_bit_cast(float4, ld_buf(Rr, kh));
            const float4 kb = __builtin_bit_cast(float4, ld_buf(Rr, kh + 16));
            const float4 va = __builtin_bit_cast(float4, ld_buf(Rr, vh));
            const float4 vb = __builtin_bit_cast(float4, ld_buf(Rr, vh + 16));
            const float4 p0 = __builtin_bit_cast(float4, ld_buf(Pr, ph));
            const float4 p1 = __builtin_bit_cast(float4, ld_buf(Pr, ph + 16));
            kq = round8<DT>(ka, kb, inv_rms_of(A, p0, p1));
            vq = round8<DT>(va, vb);
            const size_t ro = kvbase + (size_t)t * kHeadDim + 8 * ch;
            *reinterpret_cast<uint4 *>(A.kc + ro) = kq;
            *reinterpret_cast<uint4 *>(A.vc + ro) = vq;
          }
          *reinterpret_cast<uint4 *>(stk + kl * 256 + ((ch ^ (kl & 15)) << 4)) = kq;
          *reinterpret_cast<uint4 *>(stv + kl * 256 + ((ch ^ ((kl & 7) << 1)) << 4)) = vq;
        }
      }
      wave_lds_sync();   // the stage is complete before any lane reads it
      if constexpr (DB) issue(lk, lv, t0 + 2 * kRound);   // the set's next step travels during two steps
      else if (t0 + kRound < cend) issue(lk, lv, t0 + kRound);   // the next step travels during this one

      // scores: two 16-key tiles per query tile
      uint4 ka[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int kl = kt * 16 + n16, ch = 4 * s + j4;
          ka[kt][s] = lds_ld16(reinterpret_cast<const uint16_t *>(stk + kl * 256 + ((ch ^ (kl & 15)) << 4)));
        }
      f32x4_t sc[QT][2];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            a = mfma16x16x32<DT>(ka[kt][s], qh[qt][s], a);
            a = mfma16x16x32<DT>(ka[kt][s], ql[qt][s], a);
          }
          sc[qt][kt] = a;
        }
      // V^T operands: dims 16 dt + n16, keys {4 j4 .. 4 j4 + 3, 16 + 4 j4 .. 16 + 4 j4 + 3}
      uint4 va[8];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint2 h2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kl = hh * 16 + 4 * j4 + (n16 >> 2), cq = n16 & 3;
          const int ch = 2 * dt + (cq >> 1);
          h2[hh] = lds_ld8_tr16(stv + kl * 256 + ((ch ^ ((kl & 7) << 1)) << 4) + 8 * (cq & 1));
        }
        va[dt] = make_uint4(h2[0].x, h2[0].y, h2[1].x, h2[1].y);
      }
      // online softmax per query row, then the weighted values
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int m = m0 + qt * 16 + n16, r = m / GROUP;
        const int tmax = r < k ? min(cend, L + r + 1) : 0;   // keys [.., tmax) visible to this row
        float p[8];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = t0 + kt * 16 + 4 * j4 + e;
            const float v = t < tmax ? sc[qt][kt][e] : -INFINITY;
            p[kt * 4 + e] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, xpart<16>(mx));
        mx = fmaxf(mx, xpart<32>(mx));
        const float mn = fmaxf(mrun[qt], mx);
        if (__any(mn > mrun[qt])) {
          const float corr = mn > mrun[qt] ? exp2_neg(mrun[qt] - mn) : 1.f;
          lrun[qt] *= corr;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            o[qt][dt][0] *= corr;
            o[qt][dt][1] *= corr;
            o[qt][dt][2] *= corr;
            o[qt][dt][3] *= corr;
          }
        }
        mrun[qt] = mn;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = p[e] == -INFINITY ? 0.f : exp2_neg(p[e] - mn);
          lrun[qt] += p[e];
        }
        uint4 ph, pl;
        split8<DT>(p, ph, pl);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          o[qt][dt] = mfma16x16x32<DT>(va[dt], ph, o[qt][dt]);
          o[qt][dt] = mfma16x16x32<DT>(va[dt], pl, o[qt][dt]);
        }
      }
    };
    if constexpr (DB) {
      for (; t0 < cend; t0 += 2 * kRound) {
        vstep(lk0, lv0);
        if (t0 + kRound >= cend) break;
        t0 += kRound;
        vstep(lk1, lv1);
        t0 -= kRound;
      }
    } else {
      for (; t0 < cend; t0 += kRound) vstep(lk0, lv0);
    }

    // the four waves' (m, l, O) of each query tile combined into the item's partials
    float *cbuf = reinterpret_cast<float *>(dyn);   // [wave][16 rows][kVmRow]
    const int prow = threadIdx.x >> 4, pcol = (threadIdx.x & 15) * 8;   // combine: one row, 8 dims per thread
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float l = lrun[qt];
      l = xsum<16>(l);
      l = xsum<32>(l);
      __syncthreads();   // the stages (or the previous tile's combine) are no longer read
      float *cw = cbuf + (size_t)wave * 16 * kVmRow;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4_t *>(cw + n16 * kVmRow + dt * 16 + 4 * j4) = o[qt][dt];
      if (j4 == 0) {
        s_ml[wave][0][n16] = mrun[qt];
        s_ml[wave][1][n16] = l;
      }
      __syncthreads();
      const int m = m0 + qt * 16 + prow, r = m / GROUP, h = m % GROUP;
      if (r < k) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kVmWaves; ++w) M = fmaxf(M, s_ml[w][0][prow]);
        float f[kVmWaves], lt = 0.f;
#pragma unroll
        for (int w = 0; w < kVmWaves; ++w) {
          const float mw = s_ml[w][0][prow];
          f[w] = mw == -INFINITY ? 0.f : exp2_neg(mw - M);
          lt += f[w] * s_ml[w][1][prow];
        }
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kVmWaves; ++w) {
          const float *src = cbuf + ((size_t)w * 16 + prow) * kVmRow + pcol;
          const float4 a0 = *reinterpret_cast<const float4 *>(src), a1 = *reinterpret_cast<const float4 *>(src + 4);
          acc[0] += f[w] * a0.x; acc[1] += f[w] * a0.y; acc[2] += f[w] * a0.z; acc[3] += f[w] * a0.w;
          acc[4] += f[w] * a1.x; acc[5] += f[w] * a1.y; acc[6] += f[w] * a1.z; acc[7] += f[w] * a1.w;
        }
        // one workgroup-uniform resource over the item's partials (rows of the block, chunk c)
        const uint32_t pstride = (uint32_t)kMaxChunks * GROUP * kPartStride;
        const __amdgpu_buffer_rsrc_t R = rsrc_of(A.part + ((size_t)row0 * A.nkv + g) * pstride,
                                                 (uint32_t)((k - 1) * A.nkv + 1) * pstride * 4);
        const uint32_t pb = ((uint32_t)r * A.nkv * pstride + ((uint32_t)c * GROUP + h) * kPartStride) * 4;
        st_dev4(R, pb + pcol * 4, make_float4(acc[0], acc[1], acc[2], acc[3]));
        st_dev4(R, pb + (pcol + 4) * 4, make_float4(acc[4], acc[5], acc[6], acc[7]));
        if (pcol == 0) st_dev4(R, pb + 128 * 4, make_float4(M, lt, 0.f, 0.f));
      }
    }
    }   // chunks of the item
    wait_mem();   // this thread's partial stores are performed
    __syncthreads();
    if (threadIdx.x == 0)
      s_old = __hip_atomic_fetch_add(A.mctr + (size_t)row0 * A.nkv + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_old == (uint32_t)(nch_i * nt - 1)) {   // the last item of (sequence, g): merge every row of the block
      if (nch > 0) merge_block_vm<DT, GROUP>(A, row0, k, g, nch, reinterpret_cast<float *>(dyn));
      if (threadIdx.x == 0)
        __hip_atomic_store(A.mctr + (size_t)row0 * A.nkv + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();   // LDS (stages, s_old) reused by the next item
  }
}

template <int DT, int KV, int RB, int RPW>
__global__ __launch_bounds__(256) void k_oproj(LayerArgs A) {
  uint4 wr[RPW][KV];
  load_wo<KV, RPW>(A, blockIdx.x, wr);
  if (blockIdx.x == 0) advance_lengths<false>(A);
  oproj_tile<DT, KV, RB, RPW, false>(A, blockIdx.x, wr, nullptr);
}

// chunk partials of one column after the kernel boundary (plain loads); chunk
// indices clamp to the last slot (its values are never weighted then)
struct PartPlain {
  const float *p;   // chunk 0 of the column's head
  int cs, col;      // floats per chunk, float offset of the column
  __device__ __forceinline__ void operator()(int c, float2 &ml, float4 &av, bool with_av) const {
    const float *pc = p + (size_t)min(c, kMaxChunks - 1) * cs;
    ml = *reinterpret_cast<const float2 *>(pc + 128);
    if (with_av) av = *reinterpret_cast<const float4 *>(pc + col);
  }
};

// max and sum over aligned groups of CB lanes (CB = 4, 8 or 16), result in all of them
template <int CB>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  v = fmaxf(v, dpp<kQuadSwap2>(v));
  if constexpr (CB >= 8) v = fmaxf(v, dpp<kRowHalfMirror>(v));
  if constexpr (CB >= 16) v = fmaxf(v, dpp<kRowMirror>(v));
  return v;
}
template <int CB>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  if constexpr (CB >= 8) v += dpp<kRowHalfMirror>(v);
  if constexpr (CB >= 16) v += dpp<kRowMirror>(v);
  return v;
}

// o_proj for a few rows, merging the attention partials on the way in:
// att[row][h] = sum_c w_c acc_c, w_c = 2^(m_c - M) / sum_c 2^(m_c - M) l_c over
// the chunks of (row, h), M the largest m_c, summed in chunk order
// (deterministic).  Every workgroup merges all rows into LDS.  The weights
// first: thread t < nq CB takes head t / CB and chunks t % CB + CB i, the CB
// lanes of a head combine maxima and sums with lane operations, and the
// normalised weights go to LDS.  Then thread t sums the float4 columns t, t +
// 256, ... of the output.  The partials of the first CB chunks are requested
// with the W_o rows and the row table, before the row's chunk count is known;
// the chunks past it weigh zero and their values are never used (their slots
// hold an older call's values).
// SPLIT: two workgroups share output rows: each merges and contracts one half
// of the heads, and both add into the fp32 output that the projection kernel
// zeroed (two terms onto zero: the sum is the same in either order); the
// residual comes with the first half.  The pair is b and b + 8 in each group
// of 16 workgroups, so both run on the same XCD (workgroups go round-robin
// over the 8 XCDs).
template <int DT, int KV, int RPW, int CB, bool SPLIT, int MR = 1>
__global__ __launch_bounds__(256) void k_oproj_merge(LayerArgs A) {
  extern __shared__ __align__(16) unsigned char dyn[];
  float *xs = reinterpret_cast<float *>(dyn);   // [rows][this workgroup's heads x d]
  __shared__ float s_w[MR][32][kMaxChunks];   // merge weights [row][head][chunk] (nq <= 32)
  constexpr int NS = (KV + 1) / 2;              // float4 columns per thread (nq d = 512 KV)
  const int b = blockIdx.x;
  const int hh = SPLIT ? (b >> 3) & 1 : 0;                            // head half
  const int tile = SPLIT ? (b & 7) | ((b >> 4) << 3) : b;             // output rows
  const int nqb = SPLIT ? A.nq / 2 : A.nq, h0 = hh * nqb;              // heads of this workgroup
  const int K = nqb * kHeadDim, K4 = K / 4;
  const int Kw = A.nq * kHeadDim;                                      // W_o row length
  const int t = threadIdx.x;
  const int cs = A.group * kPartStride;         // floats per chunk of a kv head
  // partial of head h, chunk c of `row` (chunk index clamped into the slots)
  auto part_of = [&](int row, int h, int c) __attribute__((always_inline)) {
    const int g = h / A.group, j = h - g * A.group;
    return A.part + (((size_t)row * A.nkv + g) * kMaxChunks * A.group + j) * kPartStride +
           (size_t)min(c, kMaxChunks - 1) * cs;
  };
  const int hq = min(t / CB, nqb - 1), cq = t % CB;   // weights: (local) head and first chunk of this thread
  const bool wt = t < nqb * CB;
  // a row's merge inputs: its table record, this thread's (m, l) and the columns of the first CB chunks
  auto merge_loads = [&](int row, int4 &rt, float2 &ml0, float4 (&av)[NS][CB]) __attribute__((always_inline)) {
    rt = A.rowtab[row];
    ml0 = *reinterpret_cast<const float2 *>(part_of(row, h0 + hq, cq) + 128);
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int q4 = min(t + 256 * s2, K4 - 1);
#pragma unroll
      for (int c = 0; c < CB; ++c)
        av[s2][c] = *reinterpret_cast<const float4 *>(part_of(row, h0 + q4 / 32, c) + (q4 % 32) * 4);
    }
  };
  // The merge inputs of the first RP rows (as many as 128 registers hold) are
  // requested before the W_o rows: a wait on a load waits on every load issued
  // before it, so they arrive in one round trip and the merges run while W_o
  // travels; rows past RP (more chunks per row) request theirs one row at a time.
  // MR: the rows one pass handles (1 for single-row calls, else kVectorRows)
  constexpr int RP = 128 / (NS * CB * 4) < 1 ? 1 : (128 / (NS * CB * 4) > MR ? MR : 128 / (NS * CB * 4));
  int4 rt_p[RP];
  float2 ml0_p[RP];
  float4 av_p[RP][NS][CB];
#pragma unroll
  for (int r = 0; r < RP; ++r)
    if (r < A.rows) merge_loads(r, rt_p[r], ml0_p[r], av_p[r]);
  __builtin_amdgcn_sched_barrier(0);
  uint4 wr[RPW][KV];
  {
    const int o0 = (tile * 4 + wave_id()) * RPW;
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
      for (int v = 0; v < KV; ++v)
        wr[i][v] = ld16_stream(A.w_o + (size_t)(o0 + i) * Kw + hh * K + (v * 64 + lane_id()) * 8);
  }
  // merge of one row in two phases, the weights (into s_w[slot]) and then the
  // columns (into xs); the prefetched rows run each phase together, so their
  // chains interleave and one barrier serves them all
  auto merge_weights = [&](int slot, int row, const int4 &rt, const float2 &ml0) __attribute__((always_inline)) {
    const int nch = chunks_of(rt.x ? rt.y + (row - seq_row0(A, seq_of(A, row))) + 1 : 0, A.split);
    float mx = cq < nch ? ml0.x : -INFINITY;
    for (int c = cq + CB; c < nch; c += CB) mx = fmaxf(mx, part_of(row, h0 + hq, c)[128]);
    const float M = group_max<CB>(mx);
    const float w0 = cq < nch ? exp2_neg(ml0.x - M) : 0.f;
    float den = w0 * (cq < nch ? ml0.y : 0.f);
    for (int c = cq + CB; c < nch; c += CB) {
      const float2 v = *reinterpret_cast<const float2 *>(part_of(row, h0 + hq, c) + 128);
      den += exp2_neg(v.x - M) * v.y;
    }
    const float inv = 1.0f / group_sum<CB>(den);
    if (wt) {
      s_w[slot][hq][cq] = w0 * inv;
      for (int c = cq + CB; c < nch; c += CB) s_w[slot][hq][c] = exp2_neg(part_of(row, h0 + hq, c)[128] - M) * inv;
    }
    return nch;
  };
  auto merge_columns = [&](int slot, int row, int nch, const float4 (&av)[NS][CB]) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const int q4 = t + 256 * s2, h = min(q4, K4 - 1) / 32;
      float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const bool ok = c < nch;
        const float w = s_w[slot][h][c];   // zero past nch
        num.x += w * (ok ? av[s2][c].x : 0.f);
        num.y += w * (ok ? av[s2][c].y : 0.f);
        num.z += w * (ok ? av[s2][c].z : 0.f);
        num.w += w * (ok ? av[s2][c].w : 0.f);
      }
      for (int c = CB; c < nch; ++c) {
        const float w = s_w[slot][h][c];
        const float4 v = *reinterpret_cast<const float4 *>(part_of(row, h0 + h, c) + (q4 % 32) * 4);
        num.x += w * v.x;
        num.y += w * v.y;
        num.z += w * v.z;
        num.w += w * v.w;
      }
      if (q4 < K4) reinterpret_cast<float4 *>(xs + (size_t)row * K)[q4] = num;
    }
  };
  int nch_p[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r)
    if (r < A.rows) nch_p[r] = merge_weights(r, r, rt_p[r], ml0_p[r]);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RP; ++r)
    if (r < A.rows) merge_columns(r, r, nch_p[r], av_p[r]);
  for (int row = RP; row < A.rows; ++row) {
    int4 rt;
    float2 ml0;
    float4 av[NS][CB];
    merge_loads(row, rt, ml0, av);
    __syncthreads();   // the previous row's weights are read
    const int nch = merge_weights(0, row, rt, ml0);
    __syncthreads();
    merge_columns(0, row, nch, av);
  }
  __syncthreads();
  // the GEMV of MR rows at a time: W_o unpacked once, the rows' reductions interleaved
  const int wave = wave_id(), lane = lane_id();
  const int o0 = (tile * 4 + wave) * RPW;
  float wf[RPW][KV * 8];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int v = 0; v < KV; ++v) unpack8<DT>(wr[i][v], wf[i] + v * 8);
  for (int r0 = 0; r0 < A.rows; r0 += MR) {
    float acc[MR][RPW];
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) {
      const int row = r0 + rr;
#pragma unroll
      for (int i = 0; i < RPW; ++i) acc[rr][i] = 0.f;
      if (row < A.rows) {
#pragma unroll
        for (int v = 0; v < KV; ++v) {
          const float4 *xp = reinterpret_cast<const float4 *>(xs + (size_t)row * K + (v * 64 + lane) * 8);
          const float4 f0 = xp[0], f1 = xp[1];
          const float x8[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
          for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[rr][i] += wf[i][v * 8 + e] * x8[e];
        }
      }
    }
#pragma unroll
    for (int rr = 0; rr < MR; ++rr)
      if (r0 + rr < A.rows) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) acc[rr][i] = wave_sum(acc[rr][i]);
      }
#pragma unroll
    for (int rr = 0; rr < MR; ++rr) {
      const int row = r0 + rr;
      if (row < A.rows && lane < RPW) {
        float val = acc[rr][0];
#pragma unroll
        for (int i = 1; i < RPW; ++i)
          if (lane == i) val = acc[rr][i];
        const size_t o = (size_t)row * A.H + o0 + lane;
        if (A.residual && hh == 0) val += cvt16<DT>(A.residual[o]);
        if (!A.rowtab[row].x) val = __builtin_nanf("");
        if (SPLIT) __hip_atomic_fetch_add(reinterpret_cast<float *>(A.out) + o, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else if (A.out_f32) reinterpret_cast<float *>(A.out)[o] = val;
        else reinterpret_cast<uint16_t *>(A.out)[o] = rne16<DT>(val);
      }
    }
  }
  if (blockIdx.x == 0) advance_lengths<false>(A);
}

// lengths advance once every workgroup has read them (rows from LDS)
__device__ void advance_lengths_lds(const LayerArgs &A, const int4 *rinfo) {
  for (int b = threadIdx.x; b < A.B; b += blockDim.x) {
    const int4 ri = rinfo[seq_row0(A, b)];
    if (ri.z > 0) {
      A.lens[ri.x] = ri.y + seq_rows(A, b);
    } else if (A.status) {
      atomicOr(A.status, (ri.x >= 0 && ri.x < A.batch_cap) ? (uint32_t)ASR_STATUS_CAPACITY : kStatusBadSlot);
    }
  }
}

template <int DT, int GROUP>
__device__ __forceinline__ void resolve_flow(const LayerArgs &A, const Pending &p, AttnShared<GROUP> &S) {
  if (threadIdx.x == 0) S.flag = p.old == (uint32_t)(p.nch - 1);
  __syncthreads();
  if (S.flag) {
    merge_group<DT, GROUP, true>(A, p.row, p.g, p.nch, S);
    signal_count(A.flow + kFlowMerged);
  }
}

// All phases of a layer call in one persistent dispatch whose workgroups are
// all resident.  Workgroup w takes projection tile w, attention item w and
// o_proj tile w (and every G-th after them).  The weights of its projection
// tile are its first loads; the K/V of its first item and its W_o rows are
// requested as soon as its projection results are stored, so they travel
// while the phases wait only for the data they consume: an item for the
// projection tiles of its heads, o_proj for the merged attention output.
// (A poll returns only after every load its wave issued before it, so no
// prefetch is issued ahead of the projection's own inputs or its signal.)
// Diagnostics build only (-DASR_FLOW_TRACE): thread 0 of each workgroup stamps
// the wall clock at numbered points of k_flow into 16 slots per workgroup just
// past the split-KV partials (the caller then allocates that much more workspace).
#ifdef ASR_FLOW_TRACE
#define FLOW_TRACE(i)                                                                          \
  do {                                                                                         \
    if (threadIdx.x == 0)                                                                      \
      reinterpret_cast<unsigned long long *>(A.part + (size_t)A.rows * A.nkv * kMaxChunks * GROUP * \
                                             kPartStride)[blockIdx.x * 16 + (i)] = wall_clock64(); \
  } while (0)
#else
#define FLOW_TRACE(i) \
  do {                \
  } while (0)
#endif

template <int DT, int KVI, int RBI, int KVO, int RBO, int GROUP>
__global__ __launch_bounds__(256) void k_flow(LayerArgs A, int tiles_a, int tiles_d) {
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ AttnShared<GROUP> SA;
  __shared__ float s_ssq[RBI][4];
  __shared__ int s_ok;
  const int G = gridDim.x, w = blockIdx.x;
  int4 *rinfo = reinterpret_cast<int4 *>(dyn);
  uint16_t *knew = reinterpret_cast<uint16_t *>(rinfo + A.rows);
  uint16_t *vnew = knew + A.n * kHeadDim;
  int *pre = reinterpret_cast<int *>(vnew + A.n * kHeadDim);

  FLOW_TRACE(0);
  __shared__ uint32_t s_epoch;
  // weights of the first projection tile: the first loads of the dispatch
  uint4 wq[4][KVI];
  if (w < tiles_a) qkv_tile_weights<KVI>(A, w, wq);
  // this call's epoch from the workgroup's start ticket (workgroup 0 also adds the
  // shortfall of the start and merge units)
  uint32_t merged = 0;
  if (threadIdx.x == 0) {
    const uint32_t add = w == 0 ? kFlowStartUnit - (uint32_t)G + 1u : 1u;
    s_epoch = __hip_atomic_fetch_add(A.flow + kFlowStarted, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >>
              kFlowStartShift;
  }
  build_item_prefix(A, pre, rinfo, SA.wsum);
  FLOW_TRACE(1);
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(A.flow + kFlowLensRead, w == 0 ? kFlowStartUnit - (uint32_t)G + 1u : 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  for (int r = 0; r < A.rows; ++r) merged += rinfo[r].z > 0 ? (uint32_t)A.nkv : 0u;
  if (w == 0 && threadIdx.x == 0 && merged < kFlowMergeUnit)
    __hip_atomic_fetch_add(A.flow + kFlowMerged, kFlowMergeUnit - merged, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t e = s_epoch;
  const int total = pre[A.rows];

  // projection
  for (int t = w; t < tiles_a; t += G) {
    if (t != w) qkv_tile_weights<KVI>(A, t, wq);
    qkv_tile<DT, KVI, RBI, true>(A, t, s_ssq, wq);
    FLOW_TRACE(2);
    signal_count(A.flow + t / kTilesPerHead);
    FLOW_TRACE(3);
  }
  // K/V of the first item and W_o of the first o_proj tile, in flight while the
  // projection results travel
  KVRegs P;
  Item it0{0, 0, 0, 1};
  if (w < total) {
    it0 = decode_item(A, w, pre);
    attn_item_loads(A, it0, rinfo, P);
  }
  uint4 wo[kRpwD][KVO];
  if (w < tiles_d) load_wo<KVO, kRpwD>(A, w, wo);
  // attention
  Pending pend{-1, 0, 0, 0u};
  for (int item = w; item < total; item += G) {
    const Item it = item == w ? it0 : decode_item(A, item, pre);
    if (item != w) attn_item_loads(A, it, rinfo, P);
    if (!wait_item_inputs(A, it, rinfo, GROUP, e, &s_ok)) return;
    FLOW_TRACE(4);
    attn_item<DT, GROUP, true>(A, it, rinfo, knew, vnew, SA, P);
    FLOW_TRACE(5);
    const Pending now = signal_item(A, it);
    if (pend.row >= 0) resolve_flow<DT, GROUP>(A, pend, SA);
    pend = now;
  }
  if (pend.row >= 0) resolve_flow<DT, GROUP>(A, pend, SA);
  FLOW_TRACE(6);
  // o_proj, once every (row, kv head) with visible keys is merged
  if (!wait_count(A, A.flow + kFlowMerged, flow_target(e, kFlowMergeUnit), &s_ok)) return;
  FLOW_TRACE(7);
  if (w == 0) {   // lengths advance once every workgroup has read them
    if (!wait_count(A, A.flow + kFlowLensRead, flow_target(e, kFlowStartUnit), &s_ok)) return;
    advance_lengths_lds(A, rinfo);
  }
  for (int t = w; t < tiles_d; t += G) {
    if (t != w) load_wo<KVO, kRpwD>(A, t, wo);
    oproj_tile<DT, KVO, RBO, kRpwD, true>(A, t, wo, rinfo);
  }
  FLOW_TRACE(8);
  FLOW_TRACE(9);
}

// ---------------------------------------------------------------- launch

constexpr int rb_for(int kv) { return kv <= 2 ? 4 : (kv <= 4 ? 2 : 1); }

size_t fused_dyn_smem(const LayerArgs &a) { return lds_attn_bytes(a.rows, a.n); }

using LayerKernel = void (*)(LayerArgs);

// One phase kernel.  With diagnostics events (ev != NULL, 6 entries) the kernel
// is launched with hipExtLaunchKernelGGL, which stamps its own start and end
// into ev[2 phase] and ev[2 phase + 1].
hipError_t launch_phase(LayerKernel kern, dim3 grid, dim3 block, unsigned lds, hipStream_t s, hipEvent_t *ev,
                        int phase, const LayerArgs &a) {
  if (!kern) return hipErrorInvalidValue;
  if (ev)
    hipExtLaunchKernelGGL(kern, grid, block, lds, s, ev[2 * phase], ev[2 * phase + 1], 0u, a);
  else
    hipLaunchKernelGGL(kern, grid, block, lds, s, a);
  return hipGetLastError();
}

// eight waves (two per SIMD: twice the loads in flight per CU) while a wave's
// operand batch fits its registers, else four
int qkv_mfma_waves(int kq) { return kq <= 16 ? 8 : 4; }

// a matrix-core projection kernel and the dynamic LDS bytes it is launched with
struct MfmaKernel {
  LayerKernel fn;
  unsigned lds;
};

// LX / LW instances stage each wave's operand lines through LDS: 16 KB (x, then
// W) or 8 KB (W_o) per wave
template <int DT, bool MIX, int NTL>
MfmaKernel pick_qkv_mfma_t(int kq) {
  switch (kq) {
    case 4: return {k_qkv_mfma<DT, 4, 8, false, MIX, NTL>, 0};
    case 8: return {k_qkv_mfma<DT, 8, 8, true, MIX, NTL>, 8 * 16384};
    case 12: return {k_qkv_mfma<DT, 12, 8, false, MIX, NTL>, 0};
    case 16: return {k_qkv_mfma<DT, 16, 8, true, MIX, NTL>, 8 * 16384};
    case 20: return {k_qkv_mfma<DT, 20, 4, false, MIX, NTL>, 0};
    case 24: return {k_qkv_mfma<DT, 24, 4, false, MIX, NTL>, 0};
    case 28: return {k_qkv_mfma<DT, 28, 4, false, MIX, NTL>, 0};
    case 32: return {k_qkv_mfma<DT, 32, 4, false, MIX, NTL>, 0};
    default: return {nullptr, 0};
  }
}
// row tiles of 16 per block: one for calls of at most 16 rows (verify blocks of a
// sequence or two), else four (the weight tile's loads shared by 64 rows)
constexpr int qkv_row_tiles(int rows, bool mix) { return !mix && rows <= 16 ? 1 : 4; }
template <int DT>
MfmaKernel pick_qkv_mfma(int kq, bool mix, int ntl) {
  if (mix) return pick_qkv_mfma_t<DT, true, 4>(kq);
  return ntl == 1 ? pick_qkv_mfma_t<DT, false, 1>(kq) : pick_qkv_mfma_t<DT, false, 4>(kq);
}

template <int DT, bool MIX>
MfmaKernel pick_oproj_mfma_t(int kq) {
  switch (kq) {
    case 4: return {k_oproj_mfma<DT, 4, 8, false, MIX>, 0};
    case 8: return {k_oproj_mfma<DT, 8, 8, false, MIX>, 0};
    case 12: return {k_oproj_mfma<DT, 12, 8, false, MIX>, 0};
    case 16: return {k_oproj_mfma<DT, 16, 8, true, MIX>, 8 * 8192};
    case 20: return {k_oproj_mfma<DT, 20, 8, false, MIX>, 0};
    case 24: return {k_oproj_mfma<DT, 24, 8, false, MIX>, 0};
    case 28: return {k_oproj_mfma<DT, 28, 8, false, MIX>, 0};
    case 32: return {k_oproj_mfma<DT, 32, 8, false, MIX>, 0};
    default: return {nullptr, 0};
  }
}
template <int DT>
MfmaKernel pick_oproj_mfma(int kq, bool mix) {
  return mix ? pick_oproj_mfma_t<DT, true>(kq) : pick_oproj_mfma_t<DT, false>(kq);
}

template <int DT>
LayerKernel pick_attn(int group, bool mix, bool paged) {
#define ASR_PICK_ATTN(G)                                                              \
  case G:                                                                             \
    if (paged) return mix ? k_attn<DT, G, true, true> : k_attn<DT, G, false, true>;  \
    return mix ? k_attn<DT, G, true> : k_attn<DT, G>;
  switch (group) {
    ASR_PICK_ATTN(1) ASR_PICK_ATTN(2) ASR_PICK_ATTN(4) ASR_PICK_ATTN(8)
#undef ASR_PICK_ATTN
    default: return nullptr;
  }
}

template <int DT>
LayerKernel pick_attn_few(int group, bool paged) {
  // eight waves (two per SIMD) while the registers of a group allow, else four;
  // two steps of every wave requested before any arithmetic
  switch (group) {
    case 1: return paged ? k_attn_few<DT, 1, 8, 2, true> : k_attn_few<DT, 1, 8, 2>;
    case 2: return paged ? k_attn_few<DT, 2, 8, 2, true> : k_attn_few<DT, 2, 8, 2>;
    case 4: return paged ? k_attn_few<DT, 4, 4, 2, true> : k_attn_few<DT, 4, 4, 2>;
    case 8: return paged ? k_attn_few<DT, 8, 4, 2, true> : k_attn_few<DT, 8, 4, 2>;
    default: return nullptr;
  }
}

int few_waves(int group) { return group <= 2 ? 8 : 4; }

// the partials of as many chunks as the host expects (4, 8, or 16 while two
// float4 columns per thread keep that within registers) requested at once
template <int DT, int MR>
LayerKernel pick_oproj_merge_t(int kvo, int nch_host, bool split) {
  const int cb = nch_host <= 4 ? 4 : (nch_host > 8 && kvo <= 4 ? 16 : 8);
  if (split) {   // each workgroup: half the heads (kvo / 2 float8 columns per lane), two output rows per wave
    switch (kvo / 2) {
#define ASR_PICK_OPROJ_HALF(K) \
      case K: return cb == 4 ? k_oproj_merge<DT, K, 2, 4, true, MR> : k_oproj_merge<DT, K, 2, 8, true, MR>;
      ASR_PICK_OPROJ_HALF(1) ASR_PICK_OPROJ_HALF(2) ASR_PICK_OPROJ_HALF(3) ASR_PICK_OPROJ_HALF(4)
#undef ASR_PICK_OPROJ_HALF
      default: return nullptr;
    }
  }
  switch (kvo) {
#define ASR_PICK_OPROJ_MERGE(K) \
    case K: return cb == 4 ? k_oproj_merge<DT, K, kRpwD, 4, false, MR> : cb == 16 ? k_oproj_merge<DT, K, kRpwD, 16, false, MR> : k_oproj_merge<DT, K, kRpwD, 8, false, MR>;
#define ASR_PICK_OPROJ_MERGE8(K) \
    case K: return cb == 4 ? k_oproj_merge<DT, K, kRpwD, 4, false, MR> : k_oproj_merge<DT, K, kRpwD, 8, false, MR>;
    ASR_PICK_OPROJ_MERGE(1) ASR_PICK_OPROJ_MERGE(2) ASR_PICK_OPROJ_MERGE(3) ASR_PICK_OPROJ_MERGE(4)
    ASR_PICK_OPROJ_MERGE8(5) ASR_PICK_OPROJ_MERGE8(6) ASR_PICK_OPROJ_MERGE8(7) ASR_PICK_OPROJ_MERGE8(8)
#undef ASR_PICK_OPROJ_MERGE
#undef ASR_PICK_OPROJ_MERGE8
    default: return nullptr;
  }
}
// single-row calls (bs1 decode) keep the one-row pass: its GEMV is not widened
template <int DT>
LayerKernel pick_oproj_merge(int kvo, int nch_host, bool split, bool one_row) {
  return one_row ? pick_oproj_merge_t<DT, 1>(kvo, nch_host, split) : pick_oproj_merge_t<DT, kVectorRows>(kvo, nch_host, split);
}

// (mixed calls: never single-token-only, so no NT instance)
template <int DT>
LayerKernel pick_attn_waves(int group, bool nt, bool f8, bool mix = false, bool pg = false) {
#define ASR_PICK_WAVES(G) \
  case G: \
    if (pg) return f8 ? nullptr : (mix ? k_attn_waves<DT, G, false, false, true, true> \
                                       : (nt ? k_attn_waves<DT, G, true, false, false, true> \
                                             : k_attn_waves<DT, G, false, false, false, true>)); \
    return mix ? (f8 ? k_attn_waves<DT, G, false, true, true> : k_attn_waves<DT, G, false, false, true>) \
               : f8 ? (nt ? k_attn_waves<DT, G, true, true> : k_attn_waves<DT, G, false, true>) \
                    : (nt ? k_attn_waves<DT, G, true, false> : k_attn_waves<DT, G, false, false>);
  switch (group) {
    ASR_PICK_WAVES(2) ASR_PICK_WAVES(4)
    default: return nullptr;
  }
#undef ASR_PICK_WAVES
}

// query tiles of 16 rows for GROUP * k query rows per (sequence, kv head); 0: no instance
int vmfma_tiles(int group, int n) {
  const int m = group * n;
  return m <= 16 ? 1 : (m <= 32 ? 2 : 0);
}

// two register sets when a chunk gives each wave more than one step
bool vmfma_double_buffer(const LayerArgs &a) {
  return a.split > kVmWaves * kVmStep;
}

template <int DT>
LayerKernel pick_attn_vmfma(int group, int qt, bool db, int nt) {
#define ASR_PICK_VMFMA(G) \
  case G: return qt != 1 ? nullptr                                                                      \
                 : nt == 1 ? (db ? k_attn_vmfma<DT, G, 1, true, 1> : k_attn_vmfma<DT, G, 1, false, 1>) \
                           : (db ? k_attn_vmfma<DT, G, 1, true, 2> : k_attn_vmfma<DT, G, 1, false, 2>);
  switch (group) {
    ASR_PICK_VMFMA(2) ASR_PICK_VMFMA(4) ASR_PICK_VMFMA(8)
    default: return nullptr;
  }
#undef ASR_PICK_VMFMA
}

template <int DT>
LayerKernel pick_qkv(int kvi, bool one_row) {
  switch (kvi) {
#define ASR_PICK_QKV(K) \
    case K: return one_row ? k_qkv<DT, K, 1> : k_qkv<DT, K, rb_for(K)>;
    ASR_PICK_QKV(1) ASR_PICK_QKV(2) ASR_PICK_QKV(3) ASR_PICK_QKV(4)
    ASR_PICK_QKV(5) ASR_PICK_QKV(6) ASR_PICK_QKV(7) ASR_PICK_QKV(8)
#undef ASR_PICK_QKV
    default: return nullptr;
  }
}

template <int DT>
LayerKernel pick_oproj(int kvo, bool one_row) {
  switch (kvo) {
#define ASR_PICK_OPROJ(K) \
    case K: return one_row ? k_oproj<DT, K, 1, kRpwD> : k_oproj<DT, K, rb_for(K), kRpwD>;
    ASR_PICK_OPROJ(1) ASR_PICK_OPROJ(2) ASR_PICK_OPROJ(3) ASR_PICK_OPROJ(4)
    ASR_PICK_OPROJ(5) ASR_PICK_OPROJ(6) ASR_PICK_OPROJ(7) ASR_PICK_OPROJ(8)
#undef ASR_PICK_OPROJ
    default: return nullptr;
  }
}

template <int DT>
hipError_t layer_multi(const LayerArgs &a, int attn_grid, hipStream_t s, hipEvent_t *ev) {
  hipError_t e;
  if (a.mfma) {
    // contraction quarters of 32-wide steps: H / 128 (QKV) and nq d / 128 (o_proj)
    const int ntl = qkv_row_tiles(a.rows, a.qo_n != 0);
    const int rtiles = (a.rows + 16 * ntl - 1) / (16 * ntl);
    const MfmaKernel kq = pick_qkv_mfma<DT>(a.H / 128, a.qo_n != 0, ntl);
    if ((e = launch_phase(kq.fn, dim3(a.nqkv / 16 * rtiles), dim3(qkv_mfma_waves(a.H / 128) * kWave), kq.lds, s, ev,
                          0, a)) != hipSuccess)
      return e;
  } else {
    if ((e = launch_phase(pick_qkv<DT>(a.H / 512, a.rows == 1), dim3(a.nqkv / (4 * kRpwA)), dim3(256), 0, s, ev,
                          0, a)) != hipSuccess)
      return e;
  }
  if (!a.mfma) {
    // a few rows: partials only, merged by the o_proj kernel
    const unsigned lds_kv = (unsigned)(a.n * kHeadDim * 2 * sizeof(uint16_t));
    if ((e = launch_phase(pick_attn_few<DT>(a.group, a.ptab != nullptr), dim3(a.rows * a.nkv * a.nch_host), dim3(few_waves(a.group) * kWave),
                          lds_kv, s, ev, 1, a)) != hipSuccess)
      return e;
    const int halves = a.oproj_split ? 2 : 1, rpw = a.oproj_split ? 2 : kRpwD;
    const unsigned lds_x = (unsigned)(a.rows * a.nq / halves * kHeadDim * sizeof(float));
    return launch_phase(pick_oproj_merge<DT>(a.nq * kHeadDim / 512, a.nch_host, a.oproj_split != 0, a.rows == 1),
                        dim3(a.H / (4 * rpw) * halves), dim3(256), lds_x, s, ev, 2, a);
  }
  if (attn_vmfma_used(a)) {
    if ((e = launch_phase(pick_attn_vmfma<DT>(a.group, 1, vmfma_double_buffer(a), a.vm_nt), dim3(attn_grid), dim3(kVmWaves * kWave),
                          lds_vmfma_bytes(a.B), s, ev, 1, a)) != hipSuccess)
      return e;
  } else if (attn_waves_used(a)) {
    if ((e = launch_phase(pick_attn_waves<DT>(a.group, a.n == 1, a.kv8 != 0, a.qo_n != 0, a.ptab != nullptr), dim3(attn_grid), dim3(256), lds_attn_waves_bytes(a.rows), s,
                          ev, 1, a)) != hipSuccess)
      return e;
  } else if ((e = launch_phase(pick_attn<DT>(a.group, a.qo_n != 0, a.ptab != nullptr), dim3(attn_grid), dim3(256), lds_attn_bytes(a.rows, a.n), s,
                               ev, 1, a)) != hipSuccess) {
    return e;
  }
  if (a.mfma) {
    const MfmaKernel ko = pick_oproj_mfma<DT>(a.nq * kHeadDim / 128, a.qo_n != 0);
    return launch_phase(ko.fn, dim3(a.H / 16 * ((a.rows + 15) / 16)), dim3(512), ko.lds, s, ev, 2, a);
  }
  return launch_phase(pick_oproj<DT>(a.nq * kHeadDim / 512, a.rows == 1), dim3(a.H / (4 * kRpwD)), dim3(256), 0, s,
                      ev, 2, a);
}

// The fused kernel is instantiated for the shapes of the pages' models only
// (hidden 1024 or 2048, 16 q heads, GQA group 2); other shapes use the
// stream-ordered kernels.
bool fused_supported(const LayerArgs &a) {
  return (a.H == 1024 || a.H == 2048) && a.nq == 16 && a.group == 2;
}

template <int DT, int KVI>
hipError_t fused_launch(const LayerArgs &a, int grid, hipStream_t s, hipEvent_t *ev) {
  constexpr int KVO = 4;  // nq d = 2048
  auto kern = a.rows == 1 ? k_flow<DT, KVI, 1, KVO, 1, 2> : k_flow<DT, KVI, rb_for(KVI), KVO, rb_for(KVO), 2>;
  const int tiles_a = a.nqkv / (4 * kRpwA);
  const int tiles_d = a.H / (4 * kRpwD);
  if (ev)
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(256), fused_dyn_smem(a), s, ev[0], ev[5], 0u, a, tiles_a, tiles_d);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), fused_dyn_smem(a), s, a, tiles_a, tiles_d);
  return hipGetLastError();
}

template <int DT>
hipError_t layer_fused(const LayerArgs &a, int grid, hipStream_t s, hipEvent_t *ev) {
  if (a.H == 1024) return fused_launch<DT, 2>(a, grid, s, ev);
  return fused_launch<DT, 4>(a, grid, s, ev);
}

template <int DT, int KVI>
int occupancy_fused(size_t dyn) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_flow<DT, KVI, rb_for(KVI), 4, rb_for(4), 2>, 256,
                                                   dyn) != hipSuccess)
    return 0;
  return per_cu;
}

}  // namespace

hipError_t launch_layer_multi(const LayerArgs &a, int dtype, int attn_grid, hipStream_t s, hipEvent_t *ev) {
  return dtype == ASR_BF16 ? layer_multi<ASR_BF16>(a, attn_grid, s, ev) : layer_multi<ASR_F16>(a, attn_grid, s, ev);
}

bool layer_fused_supported(const LayerArgs &a) { return fused_supported(a); }

hipError_t launch_layer_fused(const LayerArgs &a, int dtype, int grid, hipStream_t s, hipEvent_t *ev) {
  return dtype == ASR_BF16 ? layer_fused<ASR_BF16>(a, grid, s, ev) : layer_fused<ASR_F16>(a, grid, s, ev);
}

// Largest grid of the fused kernel that is co-resident on the device: blocks
// per CU from the occupancy calculator times the CU count.
int fused_max_grid(int dtype, int H, size_t dyn_smem, int cus) {
  int per_cu;
  if (dtype == ASR_BF16) per_cu = H == 1024 ? occupancy_fused<ASR_BF16, 2>(dyn_smem) : occupancy_fused<ASR_BF16, 4>(dyn_smem);
  else per_cu = H == 1024 ? occupancy_fused<ASR_F16, 2>(dyn_smem) : occupancy_fused<ASR_F16, 4>(dyn_smem);
  return per_cu > 0 ? per_cu * cus : 0;
}

size_t layer_dyn_smem(const LayerArgs &a) { return fused_dyn_smem(a); }

// verify blocks of more than a few rows whose query rows per kv head fit two
// tiles: one K/V stream per (sequence, kv head) on the matrix cores (the
// per-row merge takes two or more q heads per kv head)
int attn_vmfma_tiles(int group, int n) { return vmfma_tiles(group, n); }

bool attn_vmfma_used(const LayerArgs &a) {
  return a.mfma && !a.qo_n && a.n > 1 && a.group >= 2 && !a.kv8 && !a.ptab && vmfma_tiles(a.group, a.n) > 0;
}

// Resident workgroups of the verify attention kernel for B sequences (blocks per
// CU from the occupancy calculator times the CU count).
int attn_vmfma_grid(int dtype, int group, int n, int B, int cus) {
  // one query tile per work item; both register-set variants hold one workgroup per CU
  if (vmfma_tiles(group, n) <= 0) return 0;
  const LayerKernel k =
      dtype == ASR_BF16 ? pick_attn_vmfma<ASR_BF16>(group, 1, false, 1) : pick_attn_vmfma<ASR_F16>(group, 1, false, 1);
  int per_cu = 0;
  if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kVmWaves * kWave, lds_vmfma_bytes(B)) != hipSuccess ||
      per_cu <= 0)
    return 0;
  return per_cu * cus;
}

// (group 8 would hold its 8 q vectors and accumulators past the register file)
bool attn_waves_used(const LayerArgs &a) { return a.mfma && (a.group == 2 || a.group == 4); }

// Resident grid of the equal-share attention kernel: blocks per CU from the
// occupancy calculator (at the largest row table) times the CU count.
int attn_waves_grid(int dtype, int group, int cus, bool mix, bool paged) {
  // occupancy per (dtype, group, mixed, paged), computed once per process; calls from
  // several threads may each compute it, they store the same value
  static std::atomic<int> cached[2][9][2][2];
  const int di = dtype == ASR_BF16 ? 1 : 0, mi = mix ? 1 : 0, pi = paged ? 1 : 0;
  if (group != 2 && group != 4) return 0;
  int per_cu = cached[di][group][mi][pi].load(std::memory_order_relaxed);
  if (per_cu <= 0) {
    const LayerKernel k = dtype == ASR_BF16 ? pick_attn_waves<ASR_BF16>(group, !mix, false, mix, paged)
                                            : pick_attn_waves<ASR_F16>(group, !mix, false, mix, paged);
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, 256, lds_attn_waves_bytes(kMaxLayerRows)) !=
                  hipSuccess || per_cu <= 0)
      return 0;
    cached[di][group][mi][pi].store(per_cu, std::memory_order_relaxed);
  }
  return per_cu * cus;
}

}  // namespace asr
