// Matrix-core building blocks of the tree-verify kernels (gfx950, bf16,
// head_dim 128): the LDS tile layout, one wavefront's share of a tile
// (S^T = K . Q^T, online softmax, O^T += V^T . P^T), and the q fragments.
//
// A wavefront owns 32 query rows (tree nodes) and a 32-token slice of a
// tile held in LDS.  S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 gives each
// lane one query column, so the softmax row statistics are lane-local (plus
// one exchange between the two lane halves), and P^T feeds the PV product's
// B operand straight from the accumulators.  The softmax runs in base 2 (q
// is pre-scaled by scale*log2 e) and the running max only moves when a
// tile's max exceeds it by more than kSlack, which skips most rescales of the
// output accumulators.
#pragma once

#include "common.h"

namespace ta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr int kD = 128;
// LDS tiles are row-major (one token per row) with padded rows: 16 lanes that
// read one 16-byte chunk from 16 consecutive K rows, or one 64-bit transpose
// read from 4 consecutive V rows x 32 bytes, land in distinct banks, and every
// access is a lane-constant address plus an immediate offset.  A stage holds
// the K rows of its tokens followed by their V rows.
constexpr int kKRow = 256 + 16;
constexpr int kVRow = 256 + 32;
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kSlack = 8.0f;  // log2 units: p <= 2^8 before a rescale

// Workgroup barrier that orders LDS only: LDS writes before it are visible to
// every wavefront after it, while global loads already issued stay in flight
// (a plain __syncthreads also waits for those).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// max(x, x of lane ^ 32) on the VALU: v_permlane32_swap exchanges the upper
// lane half of one copy of x with the lower half of another, so that in every
// lane the two results hold x of that lane and x of lane ^ 32 (in either
// order).  One VALU instruction where a shuffle is an LDS permute round trip.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// x + x of lane ^ 32 the same way (the sum is commutative, so both lanes of
// a pair get the same bits).
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r =
      __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ f32x16 mfma(const u32x4& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// gfx950 transpose read: within each group of 16 lanes, lane a points at four
// consecutive 16-bit values E[a][0..3]; lane i receives E[4k + i/4][i%4] for
// k = 0..3.  With lane a = 4k + r pointing at row (t0 + k), columns
// d0 + 4r .. d0 + 4r + 3 of a row-major tile, lane i gets column d0 + i of
// rows t0 .. t0+3: a column slice of V, as the PV operand needs it.
__device__ __forceinline__ v4i16 ds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
}

struct WaveState {
  f32x16 o[4];  // O^T, d tiles of 32: lane owns query column, rows = d
  float m, l;   // running max (log2 units) and this lane half's running sum
};

__device__ __forceinline__ void reset(WaveState& st) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) st.o[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Lane-constant LDS offsets of a wavefront that owns tokens 32*slice ..
// 32*slice+31 of a stage whose K rows take k_bytes.
struct LaneOffs {
  int k;     // K operand: row 32*slice + lane%32, chunk lane/32 (+32 bytes per k-step)
  int v;     // V transpose read: see ds_read_tr
  int base;  // first token of the slice
  int g;     // lane half
};

__device__ __forceinline__ LaneOffs lane_offsets(int lane, int slice, int k_bytes) {
  LaneOffs L;
  const int g = lane >> 5, r32 = lane & 31;
  const int grp = lane >> 4, a = lane & 15;
  L.base = 32 * slice;
  L.g = g;
  L.k = (L.base + r32) * kKRow + g * 16;
  L.v = k_bytes + (L.base + 4 * (grp >> 1) + (a >> 2)) * kVRow +
        (16 * (grp & 1) + 4 * (a & 3)) * 2;
  return L;
}

enum TileMode { kFull = 0, kPartial = 1, kTreeTile = 2, kSliceMask = 3 };

// One wavefront's 32-token slice of a stage: masked by n_valid (tokens of the
// stage at or beyond it) in kPartial mode, by the query's ancestor bitmask
// (bit j = tree node j) in kTreeTile mode, and by bit (t - 32*slice) of the
// low 32 bits of `anc_q` for token t in kSliceMask mode.
template <int kMode>
__device__ __forceinline__ void compute_tile(WaveState& st, const u32x4 (&qf)[8],
                                             const char* stage, const LaneOffs& L, int n_valid,
                                             uint64_t anc_q) {
  f32x16 s = {};
  const char* kp = stage + L.k;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    s = mfma(*reinterpret_cast<const u32x4*>(kp + 32 * ks), qf[ks], s);
  // The V^T fragments of the PV product do not depend on the probabilities.
  // In the full-tile mode of the tile loop they are read here, so that their
  // LDS latency overlaps the softmax (the rescale branch below ends the basic
  // block, and the scheduler does not move loads across it); the masked
  // modes read them after the softmax, where their registers are free.
  v8i16 va[4][2];
  const char* vp = stage + L.v;
  auto read_v = [&]() {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v4i16 lo = ds_read_tr(vp + (16 * ks) * kVRow + 64 * dt);
        const v4i16 hi = ds_read_tr(vp + (16 * ks + 8) * kVRow + 64 * dt);
        va[dt][ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  if constexpr (kMode == kFull) read_v();
  if (kMode != kFull) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = L.base + 8 * (r >> 2) + 4 * L.g + (r & 3);
      const bool ok = kMode == kTreeTile    ? ((anc_q >> tt) & 1ull) != 0ull
                      : kMode == kSliceMask ? ((anc_q >> (tt - L.base)) & 1ull) != 0ull
                                            : tt < n_valid;
      s[r] = ok ? s[r] : -INFINITY;
    }
  }
  float tmax = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
  tmax = max_xor32(tmax);
  const float m_new = (tmax > st.m + kSlack) ? tmax : st.m;
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_use);
  f32x8 p0, p1;
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    p0[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
    p1[r] = __builtin_amdgcn_exp2f(s[r + 8] - m_use);
    psum += p0[r] + p1[r];
  }
  st.l = st.l * alpha + psum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] *= alpha;
  }
  st.m = m_new;
  const bf16x8 pk[2] = {__builtin_convertvector(p0, bf16x8), __builtin_convertvector(p1, bf16x8)};
  if constexpr (kMode != kFull) read_v();
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[dt][ks]),
                                                          pk[ks], st.o[dt], 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Swizzled stage layout (no padding), for stages filled by direct-to-LDS
// loads, which write 64 lanes x 16 bytes contiguously: row r of K (then of
// V) takes 256 bytes at r*256, and its logical 16-byte chunk c sits in slot
// c ^ swz(r).  swz gives 16 consecutive rows 16 distinct slots (conflict-free
// K operand reads, one row per lane) and 4 consecutive rows distinct slot
// quads (conflict-free transpose reads of V).
// ---------------------------------------------------------------------------
constexpr int kSwzRow = 256;

__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// Lane-constant offsets of a wavefront slice (tokens 32*slice .. +31) in a
// swizzled stage whose K rows take k_bytes.
struct SwzOffs {
  int k_row;   // byte offset of this lane's K row
  int k_x;     // 16 * (lane half ^ swz(row)): k-step ks reads slot bytes (32 ks) ^ k_x
  int v_lo;    // transpose read, first 8 rows of a 16-row k-step: row offset + in-chunk byte
  int v_hi;    // ... last 8 rows
  int vx_lo;   // 16 * (chunk ^ swz(row)) for dt = 0; dt adds ^ 64 dt
  int vx_hi;
  int base;    // first token of the slice
  int g;
};

__device__ __forceinline__ SwzOffs swz_offsets(int lane, int slice, int k_bytes) {
  SwzOffs L;
  const int g = lane >> 5, r32 = lane & 31;
  const int grp = lane >> 4, a = lane & 15;
  L.base = 32 * slice;
  L.g = g;
  const int rk = L.base + r32;
  L.k_row = rk * kSwzRow;
  L.k_x = 16 * (g ^ swz(rk));
  const int t = L.base + 4 * (grp >> 1) + (a >> 2);  // + 16 ks (+ 8 for hi)
  const int c0 = 2 * (grp & 1) + ((a & 3) >> 1);     // logical chunk for dt = 0
  const int within = 8 * (a & 1);
  L.v_lo = k_bytes + t * kSwzRow + within;
  L.v_hi = L.v_lo + 8 * kSwzRow;
  L.vx_lo = 16 * (c0 ^ swz(t));
  L.vx_hi = 16 * (c0 ^ swz(t + 8));
  return L;
}

// compute_tile for a swizzled stage; bit (t - base) of `mask` keeps token t.
// The q fragments are read from LDS: k-step ks at qfrag[64 ks] (u32x4 units).
__device__ __forceinline__ void compute_tile_swz(WaveState& st, const u32x4* qfrag,
                                                 const char* stage, const SwzOffs& L,
                                                 uint32_t mask) {
  f32x16 s = {};
  const char* kp = stage + L.k_row;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    s = mfma(*reinterpret_cast<const u32x4*>(kp + ((32 * ks) ^ L.k_x)), qfrag[64 * ks], s);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int tt = 8 * (r >> 2) + 4 * L.g + (r & 3);
    s[r] = ((mask >> tt) & 1u) ? s[r] : -INFINITY;
  }
  float tmax = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float m_new = (tmax > st.m + kSlack) ? tmax : st.m;
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_use);
  f32x8 p0, p1;
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    p0[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
    p1[r] = __builtin_amdgcn_exp2f(s[r + 8] - m_use);
    psum += p0[r] + p1[r];
  }
  st.l = st.l * alpha + psum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] *= alpha;
  }
  st.m = m_new;
  const bf16x8 pk[2] = {__builtin_convertvector(p0, bf16x8), __builtin_convertvector(p1, bf16x8)};
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const char* vlo = stage + L.v_lo + (L.vx_lo ^ (64 * dt));
    const char* vhi = stage + L.v_hi + (L.vx_hi ^ (64 * dt));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const v4i16 lo = ds_read_tr(vlo + 16 * ks * kSwzRow);
      const v4i16 hi = ds_read_tr(vhi + 16 * ks * kSwzRow);
      const v8i16 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pk[ks],
                                                          st.o[dt], 0, 0, 0);
    }
  }
}

// Merge another wavefront's state for the same query columns into st.
__device__ __forceinline__ void merge_state(WaveState& st, const float* o1, float m1, float l1,
                                            int lane) {
  const float M = fmaxf(st.m, m1);
  const float Mu = M == -INFINITY ? 0.f : M;
  const float w0 = __builtin_amdgcn_exp2f(st.m - Mu);
  const float w1 = __builtin_amdgcn_exp2f(m1 - Mu);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[dt][r] = st.o[dt][r] * w0 + o1[(dt * 16 + r) * 64 + lane] * w1;
  st.l = st.l * w0 + l1 * w1;
  st.m = M;
}


// Write only O^T (64 x 64 floats, lane-major); m and l travel separately.
__device__ __forceinline__ void park_o(const WaveState& st, float* blk, int lane) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) blk[(dt * 16 + r) * 64 + lane] = st.o[dt][r];
}

// Final result of a work item for query row q (lane's column), after the
// lane halves' sums have been combined into st.l: `out` row in bf16 when the
// item covers the whole context, else the (m, l, O) partial of its split.
__device__ __forceinline__ void write_result(const WaveState& st, const VerifyParams& p, int b,
                                             int h, int bh, int sp, int nsplit, int q, int T,
                                             bool row_real, int g) {
  if (nsplit == 1) {
    if (q < T) {
      uint16_t* orow = static_cast<uint16_t*>(p.out) + (((size_t)b * T + q) * p.H + h) * kD;
      const float inv = (row_real && st.l > 0.f) ? 1.0f / st.l : 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const f32x4 v4 = {st.o[dt][4 * rb] * inv, st.o[dt][4 * rb + 1] * inv,
                            st.o[dt][4 * rb + 2] * inv, st.o[dt][4 * rb + 3] * inv};
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * rb + 4 * g) =
              __builtin_bit_cast(u32x2, __builtin_convertvector(v4, bf16x4));
        }
    }
  } else if (row_real) {
    const size_t row = ((size_t)bh * p.splits + sp) * T + q;
    float* orow = p.ws_o + row * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * rb + 4 * g) =
            f32x4{st.o[dt][4 * rb], st.o[dt][4 * rb + 1], st.o[dt][4 * rb + 2],
                  st.o[dt][4 * rb + 3]};
    if (g == 0) p.ws_ml[row] = float2{st.m, st.l};
  }
}

}  // namespace ta
