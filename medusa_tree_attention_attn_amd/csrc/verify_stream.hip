// Tree-verify attention on gfx950 matrix cores, persistent form (bf16,
// head_dim 128).
//
// What it computes is defined in tree_attn.h: every tree node attends to the
// sequence's paged KV cache plus its own ancestors, RoPE at ctx_len + depth
// (vLLM issue #1171: several new tokens over a paged cache under a tree mask;
// TensorRT-LLM issue #1946: position offsets; LMDeploy PR #1231: TreeMask over
// split-KV Flash Decoding).
//
// One workgroup of eight wavefronts per CU, resident for the whole launch.
// A unit of work is one (sequence, head, context split); units are ranked
// longest context first.  Workgroup w starts with unit w and takes each
// further unit from a counter in the workspace when three jobs of its
// current unit remain, so the CU that finishes first takes the next unit and
// the launch ends with the short units spread over the CUs.  The workgroup
// that leaves last puts the counter back to zero.
//
// A unit is a sequence of jobs: its context in jobs of 128 tokens (eight
// 16-token pages), then (split 0 only) the tree block as a job of 64 keys.
// Jobs stream through one register tile per thread and an LDS double buffer:
// while job g is computed out of LDS, job g+1 is in flight from HBM.  The
// job sequence runs on across unit boundaries: the next unit's tree rows,
// page ids and rotated q are fetched while the current unit still streams,
// so a unit's start costs no idle memory round trip.
//
// Wavefront (qt, quarter) owns query rows 32*qt .. 32*qt+31 and the 32-token
// slice `quarter` of each job (the tree job has slices 0 and 1); the four
// quarters' softmax states are merged through LDS at the end of the unit.
// Jobs go from HBM straight into LDS (direct-to-LDS loads into a swizzled
// layout), so no register tile or store phase sits between load and use.  The tree keys are rotated with the fixed-order fp32 arithmetic
// and rounded to bf16 exactly as the commit stores them.
#include "launch.h"
#include "mfma_tile.h"
#include "plan.h"

namespace ta {
namespace {

constexpr int kSThreads = 512;
constexpr int kJob = 128;                           // context tokens per job (8 pages)
constexpr int kJKBytes = kJob * kSwzRow;            // K rows of a stage (32 KB)
constexpr int kJStage = 2 * kJKBytes;               // K then V rows (64 KB)
constexpr int kQBufU4 = 2 * 8 * 64;                 // q fragments of a unit (u32x4 units)
constexpr int kPagesMax = kMaxSplitTokens / kPage;  // page ids of one split
constexpr int kAhead = 3;                           // jobs left when the next unit is taken
// Cache-policy operand of the direct-to-LDS loads: non-temporal (the data is
// read once).
constexpr int kNt = 2;
constexpr int kParkO = 64 * 64;                     // O^T of one wavefront (floats)
static_assert(2 * kJStage + 2 * kPagesMax * 4 + kQBufU4 * 16 + 4 * 2 * 64 * 4 + 16 <= 163840,
              "LDS budget");
static_assert(4 * kParkO * 4 <= kJStage, "merge area");
static_assert(kPagesMax <= kSThreads, "one page id per thread");

// Phases of the next unit's preparation.
enum NextPhase {
  kIdle = 0,       // nothing requested
  kGrabbed = 1,    // thread 0 holds the counter value
  kPublished = 2,  // the value is in LDS (readable after the next barrier)
  kMeta = 3,       // its ctx_len, tree rows, page ids and q rows are in flight
  kPages = 4,      // page ids and raw q in LDS (usable after the next barrier)
  kReady = 5,      // its jobs can be loaded
  kNone = 6        // no unit left
};

// Uniform description of a unit.
struct Unit {
  int b, h, hk, sp;
  int ctx, c0, c1, nsplit;
  int n_ctx_jobs, n_jobs;
  int t_real, nqt;
};

// Per-lane tree data of a unit (lane = node).
struct Tree {
  uint64_t anc;  // ancestor-or-self bitmask
  int dep;       // depth (clamped to [0, T-1])
};

// What a thread fetches for a unit before its jobs can start.
struct Fetch {
  int ctx_raw;
  int par, dep;  // lane = node
  int blk;       // page id of page `tid` of the split
};

// LDS-only barrier: LDS writes done, then s_barrier.  Loads that fill the
// other stage stay in flight (a plain __syncthreads would wait for them, and
// so would a workgroup fence on the local address space, which counts the
// direct-to-LDS loads as LDS writes).  The signal fences keep the compiler
// from moving any memory access across the barrier; they emit no code.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Everything this wavefront issued has landed (including its direct-to-LDS loads).
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0070); }

__device__ __forceinline__ void decode_unit(const VerifyParams& p, int r, bool ranked,
                                            int seq_rank, int lane, int& b, int& h, int& sp) {
  r = __builtin_amdgcn_readfirstlane(r);  // uniform: keep the unit in scalar registers
  if (ranked) {
    const int j = r / p.H;
    h = r - j * p.H;
    sp = 0;
    b = __builtin_ctzll(__ballot(lane < p.B && seq_rank == j));
  } else {
    const int bh = r / p.splits;
    sp = r - bh * p.splits;
    b = bh / p.H;
    h = bh - b * p.H;
  }
}

// Fetch a unit's ctx_len, tree rows and page ids into registers.
__device__ __forceinline__ void issue_fetch(Fetch& F, const VerifyParams& p, int b, int sp,
                                            int tid, int lane) {
  const int T = p.T;
  F.ctx_raw = p.ctx_lens[b];
  F.par = lane < T ? p.tree_parent[(size_t)b * T + lane] : kPadParent;
  F.dep = lane < T ? p.tree_depth[(size_t)b * T + lane] : 0;
  const int pg = ((sp * p.chunk) >> 4) + tid;
  F.blk = (tid < kPagesMax && tid < p.chunk / kPage && pg < p.max_blocks)
              ? p.block_table[(size_t)b * p.max_blocks + pg]
              : -1;
}

// The fetched values are in: build the unit and its tree masks.  For a
// split inside the context, also publish its page ids to `pages` (visible
// after the next barrier).  Returns false when the split lies beyond the
// context.
__device__ __forceinline__ bool finish_fetch(Fetch& F, Unit& U, Tree& TRi, const VerifyParams& p,
                                             int b, int h, int sp, int* pages, int tid,
                                             int lane) {
  const int T = p.T;
  U.b = b;
  U.h = h;
  U.hk = h / (p.H / p.Hkv);
  U.sp = sp;
  U.ctx = clampi(__builtin_amdgcn_readfirstlane(F.ctx_raw), 0, p.max_ctx);
  U.nsplit = U.ctx == 0 ? 1 : (U.ctx + p.chunk - 1) / p.chunk;
  U.c0 = sp * p.chunk;
  U.c1 = min(U.ctx, U.c0 + p.chunk);
  const bool valid = sp < U.nsplit;
  const int span = valid ? U.c1 - U.c0 : 0;
  U.n_ctx_jobs = (span + kJob - 1) / kJob;
  U.n_jobs = U.n_ctx_jobs + (sp == 0 ? 1 : 0);

  const bool real = lane < T && F.par != kPadParent;
  const uint64_t real_mask = __ballot(real);
  U.t_real = real_mask == ~0ull ? 64 : __builtin_ctzll(~real_mask);
  U.nqt = U.t_real > 32 ? 2 : 1;
  const bool linked = lane < U.t_real && (lane == 0 ? F.par == -1 : (F.par >= 0 && F.par < lane));
  uint64_t anc = linked ? (1ull << lane) : 0ull;
  int up = (linked && lane > 0) ? F.par : lane;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const uint64_t a_up = __shfl(anc, up);
    const int up_up = __shfl(up, up);
    anc |= a_up;
    up = up_up;
  }
  TRi.anc = anc;
  TRi.dep = clampi(F.dep, 0, T - 1);
  if (!valid) return false;

  // A page id outside the pool reads pool page 0, as in the grid kernel: its
  // K and V rows are then finite data, scored like any other token.
  const int npages = (span + kPage - 1) / kPage;
  if (tid < npages) pages[tid] = (F.blk >= 0 && F.blk < p.num_blocks) ? F.blk : 0;
  return true;
}

// Load a unit's queries into qbuf in the MFMA fragment layout
// qbuf[qt][ks][lane] (query row 32 qt + lane%32, chunk 2 ks + lane/32 for
// ks < 4, its RoPE partner 8 + 2 (ks-4) + lane/32 for ks >= 4), rotated at
// ctx + depth, scaled by scale*log2 e and rounded to bf16; rows at or beyond
// t_real are zero.  The raw rows go to qbuf by direct-to-LDS loads (wave w:
// fragments (w/4, 2 (w%4)) and (w/4, 2 (w%4) + 1)); then thread (query row
// tid/8, chunk u = tid%8 and its partner u+8) rotates them in place.  Waits
// for every load this workgroup has in flight; the caller issues the next
// job after it.
__device__ __forceinline__ void load_q(const VerifyParams& p, const Unit& U, const Tree& TRi,
                                       u32x4* qbuf, float qscale, int tid, int lane, int wv) {
  const int T = p.T;
  {
    const int qt = wv >> 2, r = 32 * qt + (lane & 31);
    if (r < T) {
      const uint16_t* row =
          static_cast<const uint16_t*>(p.q) + (((size_t)U.b * T + r) * p.H + U.h) * kD;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ks = 2 * (wv & 3) + i;
        const int c = ks < 4 ? 2 * ks + (lane >> 5) : 8 + 2 * (ks - 4) + (lane >> 5);
        __builtin_amdgcn_global_load_lds(
            row + 8 * c, (__attribute__((address_space(3))) void*)(qbuf + (qt * 8 + ks) * 64), 16,
            0, kNt);
      }
    }
  }
  const int qr = tid >> 3, u = tid & 7;
  const int pos = U.ctx + __shfl(TRi.dep, qr);
  const f32x4* csp = reinterpret_cast<const f32x4*>(p.rope + (size_t)pos * kD + 16 * u);
  f32x4 cs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) cs[i] = csp[i];
  wait_all_loads();
  lds_barrier();
  const int qt = qr >> 5, r32 = qr & 31;
  u32x4* pa = &qbuf[(qt * 8 + (u >> 1)) * 64 + (u & 1) * 32 + r32];
  u32x4* pb = &qbuf[(qt * 8 + 4 + (u >> 1)) * 64 + (u & 1) * 32 + r32];
  const u32x4 qa = *pa, qb = *pb;
  f32x8 y1, y2;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x4 t4 = cs[w];
    const float a0 = bf16_lo(qa[w]), a1 = bf16_hi(qa[w]);
    const float b0 = bf16_lo(qb[w]), b1 = bf16_hi(qb[w]);
    y1[2 * w] = (a0 * t4[0] - b0 * t4[1]) * qscale;
    y2[2 * w] = (b0 * t4[0] + a0 * t4[1]) * qscale;
    y1[2 * w + 1] = (a1 * t4[2] - b1 * t4[3]) * qscale;
    y2[2 * w + 1] = (b1 * t4[2] + a1 * t4[3]) * qscale;
  }
  u32x4 c1 = __builtin_bit_cast(u32x4, __builtin_convertvector(y1, bf16x8));
  u32x4 c2 = __builtin_bit_cast(u32x4, __builtin_convertvector(y2, bf16x8));
  if (qr >= U.t_real) {
    c1 = u32x4{0u, 0u, 0u, 0u};
    c2 = u32x4{0u, 0u, 0u, 0u};
  }
  *pa = c1;
  *pb = c2;
}

// Issue context job k of U straight into `stage` (swizzled layout).  Wave w
// takes page w of the job; each 16-row page plane is four direct-to-LDS
// loads of 64 lanes x 16 bytes (four rows), lane l carrying logical chunk
// (l%16) ^ swz(row) of row l/16 of the quad.  V rows of a page that lies
// beyond the context are zero-filled (its K rows are masked).
__device__ __forceinline__ void issue_ctx_job(char* stage, const VerifyParams& p, const Unit& U,
                                              const int* pages, int k, int wv, int lane) {
  const uint16_t* pool = static_cast<const uint16_t*>(p.kv_pages);
  const int tok0 = U.c0 + kJob * k + 16 * wv;
  const int blk = tok0 < U.c1 ? __builtin_amdgcn_readfirstlane(pages[(kJob / kPage) * k + wv]) : -1;
  char* krows = stage + 16 * wv * kSwzRow;
  const int rq = lane >> 4;  // row within the quad
  if (blk >= 0) {
    const uint16_t* kp = pool + page_row(blk, 0, U.hk, 0, p.Hkv, kD);
    const uint16_t* vp = kp + (size_t)p.Hkv * kPage * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = (lane & 15) ^ (4 * rq + i);
      const int off = (4 * i + rq) * kD + 8 * c;
      __builtin_amdgcn_global_load_lds(
          kp + off, (__attribute__((address_space(3))) void*)(krows + i * 1024), 16, 0, kNt);
      __builtin_amdgcn_global_load_lds(
          vp + off, (__attribute__((address_space(3))) void*)(krows + kJKBytes + i * 1024), 16, 0,
          kNt);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(krows + kJKBytes + i * 1024 + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
  }
}

// After this wavefront's loads of context job k landed: zero the V rows of
// its page that lie beyond the context (the tail of the last page), so that
// masked tokens contribute exact zeros whatever the pool holds there.
__device__ __forceinline__ void zero_ctx_tail(char* stage, const Unit& U, int k, int wv,
                                              int lane) {
  const int valid = U.c1 - (U.c0 + kJob * k + 16 * wv);  // rows of page wv inside the context
  if (valid > 0 && valid < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * i + (lane >> 4) >= valid)
        *reinterpret_cast<u32x4*>(stage + kJKBytes + (16 * wv + 4 * i) * kSwzRow + 16 * lane) =
            u32x4{0u, 0u, 0u, 0u};
  }
}

// The tree job goes to LDS like a context job: K rows of nodes 0..63 (raw,
// swizzled), V rows likewise, and each node's (cos, sin) row at its position
// ctx + depth in the stage's unused rows 64..127 (nodes 0..31 after the K
// rows, nodes 32..63 after the V rows, 512 bytes each).  Wave w loads K and
// V row quads 2w and 2w+1 and the (cos, sin) rows of nodes 8w .. 8w+7.
// Rows of nodes at or beyond t_real are not loaded.
__device__ __forceinline__ char* tree_cs_row(char* stage, int j) {
  return stage + (j < 32 ? 0 : kJKBytes) + 64 * kSwzRow + (j & 31) * 512;
}

__device__ __forceinline__ void issue_tree_job(char* stage, const VerifyParams& p, const Unit& U,
                                               const Tree& TRi, int wv, int lane) {
  const int T = p.T;
  const uint16_t* kn = static_cast<const uint16_t*>(p.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(p.v_new);
#pragma unroll
  for (int i2 = 0; i2 < 2; ++i2) {
    const int quad = 2 * wv + i2;
    const int j = 4 * quad + (lane >> 4);
    if (j < U.t_real) {
      const int c = (lane & 15) ^ swz(j);
      const size_t off = (((size_t)U.b * T + j) * p.Hkv + U.hk) * kD + 8 * c;
      __builtin_amdgcn_global_load_lds(
          kn + off, (__attribute__((address_space(3))) void*)(stage + quad * 1024), 16, 0, kNt);
      __builtin_amdgcn_global_load_lds(
          vn + off, (__attribute__((address_space(3))) void*)(stage + kJKBytes + quad * 1024), 16,
          0, kNt);
    }
  }
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const int pair = 4 * wv + i4;
    const int j = 2 * pair + (lane >> 5);
    const int dep_j = __shfl(TRi.dep, j);
    if (j < U.t_real) {
      const float* src = p.rope + (size_t)(U.ctx + dep_j) * kD + 4 * (lane & 31);
      __builtin_amdgcn_global_load_lds(
          src, (__attribute__((address_space(3))) void*)(tree_cs_row(stage, 2 * pair)), 16, 0, 0);
    }
  }
}

// The tree job has landed (and a barrier passed): rotate its keys in place
// (thread: node tid/8, chunk u = tid%8 and its partner u+8) with the
// fixed-order fp32 arithmetic, rounded to bf16 by v_cvt_pk_bf16_f32 (nearest
// even, as the commit rounds); rows of nodes at or beyond t_real become zero
// (K and V).
__device__ __forceinline__ void rotate_tree_job(char* stage, int t_real, int tid) {
  const int j = tid >> 3, u = tid & 7;
  char* kr = stage + j * kSwzRow;
  const int sj = swz(j);
  u32x4* pa = reinterpret_cast<u32x4*>(kr + 16 * (u ^ sj));
  u32x4* pb = reinterpret_cast<u32x4*>(kr + 16 * ((u + 8) ^ sj));
  u32x4 y1 = {0u, 0u, 0u, 0u}, y2 = {0u, 0u, 0u, 0u};
  if (j < t_real) {
    const u32x4 xa = *pa, xb = *pb;
    const f32x4* cs = reinterpret_cast<const f32x4*>(tree_cs_row(stage, j) + 64 * u);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 t4 = cs[w];
      float a1, a2, b1, b2;
      rope_pair_exact(bf16_lo(xa[w]), bf16_lo(xb[w]), t4[0], t4[1], a1, a2);
      rope_pair_exact(bf16_hi(xa[w]), bf16_hi(xb[w]), t4[2], t4[3], b1, b2);
      y1[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a1, b1}, bf16x2));
      y2[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a2, b2}, bf16x2));
    }
  }
  *pa = y1;
  *pb = y2;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int jv = 32 * i + (tid >> 4);
    if (jv >= t_real)
      *reinterpret_cast<u32x4*>(stage + kJKBytes + jv * kSwzRow + 16 * (tid & 15)) =
          u32x4{0u, 0u, 0u, 0u};
  }
}


__global__ __launch_bounds__(kSThreads, 1) void verify_stream_kernel(VerifyParams p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kJStage];
  __shared__ __attribute__((aligned(16))) u32x4 qbuf[kQBufU4];
  __shared__ __attribute__((aligned(16))) int s_pages[2][kPagesMax];
  __shared__ float s_ml[4][2][64];  // (m, l) of parked wavefront states
  __shared__ int s_next;

  const int tid0 = threadIdx.x, wv = tid0 >> 6;
  const int qt = wv >> 2, quarter = wv & 3;

  const int T = p.T;
  const int n_units = p.B * p.H * p.splits;
  const int grid = (int)gridDim.x;
  const float qscale = p.scale * kLog2e;
  const bool ranked = p.B <= 64 && p.splits == 1;

  int seq_rank = 0;  // rank of this lane's sequence by context length (longest first)
  {
    const int lane = tid0 & 63;
  if (ranked) {
    const int ctx_l = lane < p.B ? p.ctx_lens[lane] : -1;
    for (int j = 0; j < p.B; ++j) {
      const int cj = __shfl(ctx_l, j);
      seq_rank += (cj > ctx_l) || (cj == ctx_l && j < lane);
    }
  }
  }

  // U: the unit being computed (live until its rows are written); N: the
  // next one, prepared through the phases above.  The workgroup's first unit
  // is rank blockIdx.x and enters as an already published rank.
  Unit U{}, N{};
  Tree TU{}, TN{};
  Fetch F{};
  bool u_live = false;
  int pb = 1;  // s_pages buffer of U (N uses pb ^ 1)
  int nb = 0, nh = 0, nsp = 0;
  int phase = kPublished;
  uint32_t grab_v = 0;
  if (tid0 == 0) s_next = blockIdx.x;

  bool r_valid = false;  // a job is in flight to the other stage ...
  int r_n = 0, rk = 0;   // ... job rk of N (r_n) or of U
  int l_n = 0, lk = 0;   // next job to issue: job lk of N (l_n) or of U
  int k = -1;            // job of U in stage(cur); -1: none
  int cur = 0;
  uint64_t anc_q = 0;
  bool active = false, row_real = false;
  WaveState st;
  reset(st);
  __syncthreads();  // s_next

  for (;;) {
    // Lane-derived offsets are recomputed every step from an opaque copy of
    // the thread index: hoisted out of the loop they would pin ~190 VGPRs.
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int q = 32 * qt + (lane & 31);
    // ---- 1. compute job k of U out of stage(cur).
    if (k >= 0 && active) {
      const char* sg = smem + cur * kJStage;
      const SwzOffs L0 = swz_offsets(lane, quarter, kJKBytes);
      const u32x4* qfrag = qbuf + qt * 8 * 64 + lane;
      if (k < U.n_ctx_jobs) {
        const int nv = min(kJob, U.c1 - (U.c0 + kJob * k)) - 32 * quarter;
        if (nv > 0)
          compute_tile_swz(st, qfrag, sg, L0, nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u));
      } else if (quarter < 2) {
        compute_tile_swz(st, qfrag, sg, L0, (uint32_t)(anc_q >> (32 * quarter)));
      }
    }
    const bool u_done = u_live && k == U.n_jobs - 1;

    // ---- 2. next unit: the step before the barrier.
    if (phase == kGrabbed) {
      if (tid == 0) s_next = (int)grab_v;
      phase = kPublished;
    } else if (phase == kMeta) {
      phase = finish_fetch(F, N, TN, p, nb, nh, nsp, s_pages[pb ^ 1], tid, lane) ? kPages : kIdle;
    }

    // ---- 3. the job in flight lands in the other stage; one barrier.
    const bool staged = r_valid;
    const int staged_n = r_n, staged_k = rk;
    char* nxt = smem + (cur ^ 1) * kJStage;
    const bool staged_tree = staged && rk >= (r_n ? N.n_ctx_jobs : U.n_ctx_jobs);
    if (staged) {
      wait_all_loads();
      if (!staged_tree) zero_ctx_tail(nxt, r_n ? N : U, rk, wv, lane);
    }
    __syncthreads();
    if (staged_tree) {
      rotate_tree_job(nxt, r_n ? N.t_real : U.t_real, tid);
      lds_barrier();
    }

    // ---- 4. next unit: the step after the barrier.
    if (phase == kPublished) {
      const int r = s_next;
      if (r >= n_units) {
        phase = kNone;
      } else {
        decode_unit(p, r, ranked, seq_rank, lane, nb, nh, nsp);
        issue_fetch(F, p, nb, nsp, tid, lane);
        phase = kMeta;
      }
    } else if (phase == kPages) {
      phase = kReady;
    }
    const bool want = !u_live || U.n_jobs - 1 - k <= kAhead;
    if (phase == kIdle && want) {
      if (tid == 0) grab_v = (uint32_t)grid + atomicAdd(p.ws_ctr, 1u);
      phase = kGrabbed;
    }

    // ---- 5. U's last job is done: merge the four token quarters, write its
    // rows (O parks in stage(cur), before the next job is issued into it).
    if (u_done) {
      float* park = reinterpret_cast<float*>(smem + cur * kJStage);
      const int slot = 2 * qt + (quarter >> 1);  // quarters 1 -> 0 and 3 -> 2, then 2 -> 0
      if (active && (quarter & 1)) {
        park_o(st, park + slot * kParkO, lane);
        s_ml[slot][0][lane] = st.m;
        s_ml[slot][1][lane] = st.l;
      }
      lds_barrier();
      if (active && !(quarter & 1))
        merge_state(st, park + slot * kParkO, s_ml[slot][0][lane], s_ml[slot][1][lane], lane);
      lds_barrier();
      if (active && quarter == 2) {
        park_o(st, park + slot * kParkO, lane);
        s_ml[slot][0][lane] = st.m;
        s_ml[slot][1][lane] = st.l;
      }
      lds_barrier();
      if (quarter == 0) {
        const int s2 = 2 * qt + 1;
        if (active) {
          merge_state(st, park + s2 * kParkO, s_ml[s2][0][lane], s_ml[s2][1][lane], lane);
          st.l = sum_xor32(st.l);
        }
        write_result(st, p, U.b, U.h, U.b * p.H + U.h, U.sp, U.nsplit, q, T, row_real, lane >> 5);
      }
      lds_barrier();  // the merge area is about to be refilled
      u_live = false;
    }

    // ---- 6. N's first job has just landed: its queries go to qbuf first
    // (one exposed round trip per unit; qbuf is free once U's rows are out).
    if (staged && staged_n) load_q(p, N, TN, qbuf, qscale, tid, lane, wv);

    // Issue the next job: U's jobs, then N's.  Its stage is the one
    // that is not current after step 7 (stage(cur) when a job was staged
    // above, else the other one); both hold nothing needed any more.
    if (!l_n && lk >= U.n_jobs && phase == kReady) {
      l_n = 1;
      lk = 0;
    }
    r_valid = l_n ? (phase == kReady && lk < N.n_jobs) : (lk < U.n_jobs);
    if (r_valid) {
      char* dst = smem + (staged ? cur : cur ^ 1) * kJStage;
      if (lk < (l_n ? N.n_ctx_jobs : U.n_ctx_jobs))
        issue_ctx_job(dst, p, l_n ? N : U, s_pages[pb ^ l_n], lk, wv, lane);
      else
        issue_tree_job(dst, p, l_n ? N : U, l_n ? TN : TU, wv, lane);
      r_n = l_n;
      rk = lk;
      ++lk;
    }

    // ---- 7. the staged job becomes current; N's first job makes N current.
    if (staged) {
      cur ^= 1;
      k = staged_k;
      if (staged_n) {
        U = N;
        TU = TN;
        u_live = true;
        pb ^= 1;
        phase = kIdle;
        r_n = 0;
        l_n = 0;
        lds_barrier();  // rotated q visible
        anc_q = __shfl(TU.anc, q);
        active = qt < U.nqt;
        row_real = active && q < U.t_real;
        reset(st);
      }
    } else {
      k = -1;
      if (!u_live && phase == kNone) break;  // nothing left
    }
  }

  // The last workgroup out puts the counters back to zero for the next launch.
  if (tid0 == 0) {
    if (atomicAdd(p.ws_ctr + 1, 1u) == (uint32_t)grid - 1u) {
      atomicExch(p.ws_ctr, 0u);
      atomicExch(p.ws_ctr + 1, 0u);
    }
  }
}

}  // namespace


hipError_t launch_verify_stream(const VerifyParams& p, hipStream_t stream) {
  const long long units = (long long)p.B * p.H * p.splits;
  if (units <= 0 || units > 0x7FFFFFFF || p.n_cu <= 0 || !p.ws_ctr) return hipErrorInvalidValue;
  const int grid = (int)(units < p.n_cu ? units : p.n_cu);
  hipLaunchKernelGGL(verify_stream_kernel, dim3(grid), dim3(kSThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ta
