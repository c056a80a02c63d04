// Tree-verify attention on gfx950 matrix cores (bf16, head_dim 128).
//
// What it computes is defined in tree_attn.h: every tree node attends to the
// sequence's paged KV cache plus its own ancestors, RoPE at ctx_len + depth
// (vLLM issue #1171: several new tokens over a paged cache under a tree mask;
// TensorRT-LLM issue #1946: position offsets; LMDeploy PR #1231: TreeMask over
// split-KV Flash Decoding).
//
// Work item = (sequence b, query head h, context split sp); one workgroup of
// four wavefronts per item.  The split's context is streamed in tiles of 64
// tokens (four 16-token pages):
//   * each tile is loaded from HBM once, with 16-byte fully coalesced loads,
//     into registers one tile ahead, then written to an LDS double buffer;
//     every tree query of the head reads it from LDS;
//   * wavefront (qt, th) owns query rows 32*qt .. 32*qt+31 (the tree nodes)
//     and the 32-token half th of each tile;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: each lane owns one query
//     column, so the softmax row statistics are lane-local (plus one exchange
//     between the two lane halves), and P^T feeds the PV product's B operand
//     straight from the accumulators;
//   * V rows go to LDS as they are (rows past the context's end as zeros)
//     and the PV A operand is read column-wise with the gfx950 transpose
//     read (ds_read_b64_tr_b16);
//   * online softmax in base 2 (q is pre-scaled by scale*log2 e); the running
//     max only moves when a tile's max exceeds it by more than 8, which skips
//     most rescales of the output accumulators;
//   * split 0 also processes the tree block: the T new keys, rotated with the
//     fixed-order fp32 arithmetic and rounded to bf16 exactly as the commit
//     will store them, masked by per-node ancestor bitmasks built with
//     pointer doubling across the lanes of a wavefront.
// Splits of one (b, h) leave (m, l, O) partials in the workspace; a second,
// small kernel merges them.  The prologue takes three dependent memory round
// trips: the launch ranking (every sequence's ctx_len, and the tree row that
// marks small trees), then the work item's page ids, tree rows, q rows and
// tree k/v rows with the (cos, sin) rows of depths 0-7 (ctx_len is known by
// then), then the first two context tiles; the queries and the tree tile are
// rotated and the tree tile is computed while those tiles load.
#include "launch.h"
#include "mfma_tile.h"
#include "page_stream.h"
#include "plan.h"

namespace ta {
namespace {

constexpr int kTile = 64;                       // tokens per LDS tile (four pages)
constexpr int kThreads = 256;
constexpr int kKBytes = kTile * kKRow;
constexpr int kVBytes = kTile * kVRow;
constexpr int kStageBytes = kKBytes + kVBytes;
constexpr int kMaxSplitPages = kMaxSplitTokens / kPage;

// The occupancy the register budget is sized for (workgroups of 4
// wavefronts per CU).
#ifndef TA_WG_PER_CU
#define TA_WG_PER_CU 2
#endif

// One tile's worth of global data held by a thread between load and store:
// row tid/16 (of page p), 16-byte chunk tid%16, of the K and of the V plane.
struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
};

// Where the split's pages live: their physical ids were copied into LDS
// (s_pages[i] = page of tokens c0 + 16 i; an id outside the pool reads page
// 0) so the tile loop issues its KV loads without waiting on any table
// lookup.
struct Geo {
  const uint16_t* pages;
  const int* s_pages;
  int c0, hk, Hkv;
  int last_page;  // index of the split's last page in s_pages
};

// The page ids of context tile [tile0, tile0 + 64): one 16-byte LDS read of
// the four entries from base4 = min(pg0, last_page & ~3) on (pg0 is a
// multiple of four; s_pages is 16-byte aligned and holds whole groups of
// four).  The tile loop reads them before it computes the current tile, so
// that only scalar address arithmetic stands between its barrier and the
// next tile's loads.
__device__ __forceinline__ u32x4 fetch_page_ids(const Geo& G, int tile0) {
  const int pg0 = (tile0 - G.c0) >> 4;
  const int base4 = min(pg0, G.last_page & ~3);
  return *reinterpret_cast<const u32x4*>(G.s_pages + base4);
}

// Issue the loads of context tile [tile0, tile0 + 64) from its page ids.
// Pages past the split's end load its last page again (store_tile zeroes
// their rows), so the loads are unconditional and the compiler can count
// them: page pg0 + p reads entry min(pg0 + p, last_page) - base4, which lies
// in 0..3 whether or not the tile starts past the last page.  Page ids are
// uniform, so page addresses are scalar; each lane adds a constant offset.
// The KV stream is read once, so the loads carry the non-temporal hint: with
// it the kernel streams at about 6.2 TB/s in steady state, against 5.6
// without (7B-shaped batch 16: 63 against 70.5 us per launch).
__device__ __forceinline__ void issue_ctx_tile(TileRegs& R, const Geo& G, const u32x4 ids,
                                               int tile0, int tid) {
  const int pg0 = (tile0 - G.c0) >> 4;
  const int base4 = min(pg0, G.last_page & ~3);
  const int off = (tid >> 4) * kD + (tid & 15) * 8;
  const size_t v_plane = (size_t)G.Hkv * kPage * kD;
  const int i0 = __builtin_amdgcn_readfirstlane(ids[0]), i1 = __builtin_amdgcn_readfirstlane(ids[1]);
  const int i2 = __builtin_amdgcn_readfirstlane(ids[2]), i3 = __builtin_amdgcn_readfirstlane(ids[3]);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int e = min(pg0 + p, G.last_page) - base4;
    const int blk = e == 0 ? i0 : e == 1 ? i1 : e == 2 ? i2 : i3;
    const uint16_t* kp = G.pages + page_row(blk, 0, G.hk, 0, G.Hkv, kD);
    R.k[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + off));
    R.v[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + v_plane + off));
  }
}

__device__ __forceinline__ void load_ctx_tile(TileRegs& R, const Geo& G, int tile0, int tid) {
  issue_ctx_tile(R, G, fetch_page_ids(G, tile0), tile0, tid);
}

// Rows at or past n_rows (the tokens of the context's last page after its
// end) are written as zeros: their scores are masked, but a NaN left in an
// unused cache slot would still turn 0 * V into NaN in the P.V product.
__device__ __forceinline__ void store_tile(const TileRegs& R, char* stage, int n_rows, int tid) {
  char* kb = stage + (tid >> 4) * kKRow + (tid & 15) * 16;
  char* vb = stage + kKBytes + (tid >> 4) * kVRow + (tid & 15) * 16;
  const u32x4 z{0u, 0u, 0u, 0u};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const bool ok = 16 * p + (tid >> 4) < n_rows;
    *reinterpret_cast<u32x4*>(kb + 16 * p * kKRow) = ok ? R.k[p] : z;
    *reinterpret_cast<u32x4*>(vb + 16 * p * kVRow) = ok ? R.v[p] : z;
  }
}

// The tree block as a 64-token tile, and the queries.  Node j sits at
// position ctx + depth[j], and one (cos, sin) table row serves both its key
// and its query:
//   * key j = RoPE(k_new[b][j]) with the commit's fixed-order fp32
//     arithmetic, rounded to bf16 as the commit stores it; value j =
//     v_new[b][j]; nodes >= t_real are zero;
//   * query j = RoPE(q[b][j][h]) * scale * log2 e, rounded to bf16, written
//     row-major to a query buffer from which every wavefront then reads its
//     MFMA fragments (rows >= t_real are zero).
// Thread tid rotates node tid/4, dims 16*(tid%4) .. +15 and their partners
// (d + 64), of both rows; it copies V rows 16*q4 + tid/16, chunk tid%16.
// Loading q this way needs the table row once per node instead of once per
// query lane, which keeps the prologue's registers low enough to issue
// context tiles 0 and 1 together.  These rows keep the default cache policy:
// with the non-temporal hint on the q rows, the tree rows or both the
// 7B-shaped batch-16 launch took 0.6-2.6 us longer.
struct TreeRaw {
  u32x4 k[4];    // chunks 2u, 2u+1 (first half) and 8+2u, 9+2u (second half)
  u32x4 q[4];    // the same chunks of the node's query row
  u32x4 v[4];
  f32x4 cs[8];   // (cos, sin) of k = 16u .. 16u+15
};
// Tree rows past last_row (query rows past T - 1) read that row instead:
// store_tree_tile zeroes every row at or past t_real, so the loads are
// unconditional and the wavefront issues all of them without waiting on any.
__device__ __forceinline__ void load_tree_raw(TreeRaw& TR, const VerifyParams& p, int b, int h,
                                              int hk, int last_row, int tid) {
  const int T = p.T;
  const uint16_t* kn = static_cast<const uint16_t*>(p.k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(p.v_new);
  const int j = min(tid >> 2, last_row), u = tid & 3;
  const uint16_t* row = kn + (((size_t)b * T + j) * p.Hkv + hk) * kD;
  const uint16_t* qrow =
      static_cast<const uint16_t*>(p.q) + (((size_t)b * T + min(tid >> 2, T - 1)) * p.H + h) * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int off = (i >> 1) * 64 + 16 * u + 8 * (i & 1);
    TR.q[i] = *reinterpret_cast<const u32x4*>(qrow + off);
    TR.k[i] = *reinterpret_cast<const u32x4*>(row + off);
  }
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int jv = min(16 * q4 + (tid >> 4), last_row);
    TR.v[q4] = *reinterpret_cast<const u32x4*>(vn + (((size_t)b * T + jv) * p.Hkv + hk) * kD +
                                               (tid & 15) * 8);
  }
}
__device__ __forceinline__ void load_tree_rope(TreeRaw& TR, const float* rope, int pos_j, int tid) {
  const f32x4* cs = reinterpret_cast<const f32x4*>(rope + (size_t)pos_j * kD + 2 * 16 * (tid & 3));
#pragma unroll
  for (int i = 0; i < 8; ++i) TR.cs[i] = cs[i];
}
constexpr int kQRow = 256 + 16;  // query buffer row (padded as the K rows)

// The (cos, sin) rows of positions ctx .. ctx + kRopeRows - 1 (tree depths
// 0 .. kRopeRows - 1) are staged in LDS during round trip 1, when the
// launch ranking has already read ctx_len, so that the tree tile and the
// queries can be rotated as soon as round trip 1 is back; trees with deeper
// nodes read their rows from the table in round trip 2.  They sit in stage 0
// after the query buffer, which no context tile takes before the rotation.
constexpr int kRopeRows = 8;
constexpr int kRopeRowBytes = kD * 4;
constexpr int kRopeOff = kTile * kQRow;
__device__ __forceinline__ void read_tree_rope_lds(TreeRaw& TR, const char* rope_lds, int row,
                                                   int tid) {
  const f32x4* cs = reinterpret_cast<const f32x4*>(rope_lds + row * kRopeRowBytes) + 8 * (tid & 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) TR.cs[i] = cs[i];
}
__device__ __forceinline__ void store_tree_tile(char* stage, char* qbuf, const TreeRaw& TR,
                                                int t_real, float qscale, bool with_kv, int tid) {
  const int j = tid >> 2, u = tid & 3;
  u32x4 c[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  u32x4 e[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  if (j < t_real) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x4 t4 = TR.cs[4 * h2 + w];
        float y1a, y2a, y1b, y2b;
        rope_pair_exact(bf16_lo(TR.k[h2][w]), bf16_lo(TR.k[2 + h2][w]), t4[0], t4[1], y1a, y2a);
        rope_pair_exact(bf16_hi(TR.k[h2][w]), bf16_hi(TR.k[2 + h2][w]), t4[2], t4[3], y1b, y2b);
        // v_cvt_pk_bf16_f32 rounds to nearest even, as the commit's integer
        // rounding does, for every finite value.
        c[h2][w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{y1a, y1b}, bf16x2));
        c[2 + h2][w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{y2a, y2b}, bf16x2));
        float x1a, x2a, x1b, x2b;
        rope_pair_exact(bf16_lo(TR.q[h2][w]), bf16_lo(TR.q[2 + h2][w]), t4[0], t4[1], x1a, x2a);
        rope_pair_exact(bf16_hi(TR.q[h2][w]), bf16_hi(TR.q[2 + h2][w]), t4[2], t4[3], x1b, x2b);
        e[h2][w] = __builtin_bit_cast(
            uint32_t, __builtin_convertvector(f32x2{x1a * qscale, x1b * qscale}, bf16x2));
        e[2 + h2][w] = __builtin_bit_cast(
            uint32_t, __builtin_convertvector(f32x2{x2a * qscale, x2b * qscale}, bf16x2));
      }
    }
  }
  char* qr = qbuf + j * kQRow;
  *reinterpret_cast<u32x4*>(qr + 16 * (2 * u)) = e[0];
  *reinterpret_cast<u32x4*>(qr + 16 * (2 * u + 1)) = e[1];
  *reinterpret_cast<u32x4*>(qr + 16 * (8 + 2 * u)) = e[2];
  *reinterpret_cast<u32x4*>(qr + 16 * (9 + 2 * u)) = e[3];
  if (!with_kv) return;
  char* kr = stage + j * kKRow;
  *reinterpret_cast<u32x4*>(kr + 16 * (2 * u)) = c[0];
  *reinterpret_cast<u32x4*>(kr + 16 * (2 * u + 1)) = c[1];
  *reinterpret_cast<u32x4*>(kr + 16 * (8 + 2 * u)) = c[2];
  *reinterpret_cast<u32x4*>(kr + 16 * (9 + 2 * u)) = c[3];
  char* vb = stage + kKBytes + (tid >> 4) * kVRow + (tid & 15) * 16;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int jv = 16 * q4 + (tid >> 4);
    *reinterpret_cast<u32x4*>(vb + 16 * q4 * kVRow) =
        jv < t_real ? TR.v[q4] : u32x4{0u, 0u, 0u, 0u};
  }
}
// Q^T fragments of query row q for k-steps 0..7 from the query buffer: chunk
// 2*ks + g for ks < 4, its RoPE partner chunk 8 + 2*(ks-4) + g for ks >= 4.
__device__ __forceinline__ void load_q_frags(u32x4 (&qf)[8], const char* qbuf, int q, int g) {
  const char* row = qbuf + q * kQRow;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int c = ks < 4 ? 2 * ks + g : 8 + 2 * (ks - 4) + g;
    qf[ks] = *reinterpret_cast<const u32x4*>(row + 16 * c);
  }
}

// Output of an unsplit item.  Each wavefront writes its two d-tiles of the
// normalised rows as bf16 (lane = query column, four consecutive dims per
// value group) into a row-major tile in LDS; then all four wavefronts store
// whole 256-byte rows of `out`, 16 bytes per lane, instead of 8-byte pieces
// of 32 rows per instruction.  Rows q >= T are not stored; padding rows are
// zeros.
constexpr int kOutRow = 256 + 16;  // padded: the value-group writes spread over the banks
template <int d0>
__device__ __forceinline__ void stage_out(const WaveState& st, char* tile, int q, bool row_real,
                                          int g) {
  const float inv = (row_real && st.l > 0.f) ? 1.0f / st.l : 0.f;
  char* row = tile + q * kOutRow;
#pragma unroll
  for (int dt = d0; dt < d0 + 2; ++dt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const f32x4 v4 = {st.o[dt][4 * rb] * inv, st.o[dt][4 * rb + 1] * inv,
                        st.o[dt][4 * rb + 2] * inv, st.o[dt][4 * rb + 3] * inv};
      *reinterpret_cast<u32x2*>(row + 2 * (32 * dt + 8 * rb + 4 * g)) =
          __builtin_bit_cast(u32x2, __builtin_convertvector(v4, bf16x4));
    }
}
__device__ __forceinline__ void store_out(const char* tile, const VerifyParams& p, int b, int h,
                                          int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;  // 16-byte chunk c % 16 of row c / 16
    const int row = c >> 4, ch = c & 15;
    if (row < p.T)
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) +
                                (((size_t)b * p.T + row) * p.H + h) * kD + 8 * ch) =
          *reinterpret_cast<const u32x4*>(tile + row * kOutRow + 16 * ch);
  }
}

// Merge of the two token halves of a query tile, shared by its two
// wavefronts: wavefront th keeps d-tiles 2th and 2th+1 of O^T.  Each parks
// the other pair and its (m, l) in a block of 34 x 64 floats (eight
// lane-major groups of four accumulators, written and read 16 bytes per
// lane, then m and l), and after a barrier merges its own pair with the pair
// its partner parked.  The running sums are combined in one fixed order
// (th = 0's first), so both wavefronts hold the same l.
constexpr int kHalfPark = 34 * 64;  // floats per wavefront
template <int kDOther>
__device__ __forceinline__ void park_half(const WaveState& st, float* blk, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x16& o = st.o[kDOther + j];
      *reinterpret_cast<f32x4*>(blk + ((4 * j + r4) * 64 + lane) * 4) =
          f32x4{o[4 * r4], o[4 * r4 + 1], o[4 * r4 + 2], o[4 * r4 + 3]};
    }
  blk[32 * 64 + lane] = st.m;
  blk[33 * 64 + lane] = st.l;
}
template <int kTh>
__device__ __forceinline__ void merge_half(WaveState& st, const float* pblk, int lane) {
  constexpr int d_own = 2 * kTh;
  const float m1 = pblk[32 * 64 + lane], l1 = pblk[33 * 64 + lane];
  const float M = fmaxf(st.m, m1);
  const float Mu = M == -INFINITY ? 0.f : M;
  const float w_own = __builtin_amdgcn_exp2f(st.m - Mu);
  const float w_par = __builtin_amdgcn_exp2f(m1 - Mu);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(pblk + ((4 * j + r4) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        st.o[d_own + j][4 * r4 + e] = st.o[d_own + j][4 * r4 + e] * w_own + x[e] * w_par;
    }
  const float la = kTh == 0 ? st.l : l1, wa = kTh == 0 ? w_own : w_par;
  const float lb = kTh == 0 ? l1 : st.l, wb = kTh == 0 ? w_par : w_own;
  st.l = la * wa + lb * wb;
  st.m = M;
}
// Split partial of a work item: this wavefront's two d-tiles of O^T; the
// th = 0 wavefront also writes (m, l).
template <int d0>
__device__ __forceinline__ void write_partial_half(const WaveState& st, const VerifyParams& p,
                                                   int bh, int sp, int q, int T, bool row_real,
                                                   int g, bool write_ml) {
  if (!row_real) return;
  const size_t row = ((size_t)bh * p.splits + sp) * T + q;
  float* orow = p.ws_o + row * kD;
#pragma unroll
  for (int dt = d0; dt < d0 + 2; ++dt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * rb + 4 * g) =
          f32x4{st.o[dt][4 * rb], st.o[dt][4 * rb + 1], st.o[dt][4 * rb + 2], st.o[dt][4 * rb + 3]};
  if (write_ml && g == 0) p.ws_ml[row] = float2{st.m, st.l};
}

// What round trip 1 of a work item leaves: its context bounds, and the
// tree structure with one lane per node (every wavefront computes it).
struct ItemMeta {
  int ctx, nsplit, c1, npages;
  int t_real;     // real nodes (a prefix of the rows)
  uint64_t anc;   // ancestor-or-self bitmask of node `lane`
  int dep;        // depth of node `lane`
  int pos_j;      // position of node tid/4: ctx + its depth
  bool rope_lds;  // this wavefront's nodes take their (cos, sin) rows from LDS
};

// ---------------------------------------------------------------------------
// Small trees (at most kSmallTree = 2 real nodes, e.g. the one-node rows of
// a mixed batch where speculation is off for some sequences): a 32-query
// matrix-core tile would be mostly padding, so the item keeps the page
// streamer and the prologue of the tree path (page ids in LDS, rotated
// queries and the tree tile in LDS, context tiles 0 and 1 in flight in
// registers) and then consumes each context tile straight from its
// registers on the vector ALU, as the one-node decode kernel does: thread
// tid holds dims 8 (tid % 16) .. +7 of K and V of token 16 p + tid / 16 of
// the tile (p = 0..3), so lane group tid / 16 of the workgroup scores its
// four tokens against every query with dot2 sums over 16 lanes and keeps
// one online-softmax state per query.  No tile goes through LDS and no
// barrier sits in the loop; each tile's registers take the tile two ahead
// once consumed.  The tree keys join lane groups 0..7 (node 4 w + g of
// wavefront w, group g), masked by each query's ancestor bitmask.  The 16
// states of each query are merged through LDS at the end.  The item is
// routed here at launch (the tree row at index kSmallTree is padding), so
// the two paths share no registers (the kernel stays within 256 VGPRs; 8
// queries, 80 VGPRs of states beside two register tiles, spilled).  The
// vector-ALU work grows with the queries while the matrix-core tile does
// not, so the cut is at 2 nodes.  Measured on stress-shaped batches of 64
// sequences (contexts 128..8192) whose trees all have 1, 2 or 4 nodes: 672,
// 679 and 691 us on this path against 682, 686 and 686 us on the matrix
// cores; one-node trees at batch 64 624 us against 637 us for the decode
// kernel.
// ---------------------------------------------------------------------------
constexpr int kSmallTree = 2;

template <int kM>
__device__ __forceinline__ void small_tree_item(const VerifyParams& p, const Geo& G, TreeRaw& TR,
                                                const ItemMeta& M, char* smem, int n_tiles,
                                                int c0, int b, int h, int sp, int tid) {
  const int lane = tid & 63, wv = tid >> 6, grp = lane >> 4, dc = lane & 15;
  const int T = p.T;
  const int c1 = M.c1, nsplit = M.nsplit, t_real = M.t_real;
  const uint64_t anc = M.anc;
  // Round trip 2 as on the matrix-core path: context tiles 0 and 1 (and the
  // (cos, sin) rows when they are not in LDS); the rotated queries go to
  // stage 0, the tree tile to stage 1 (no context tile goes through LDS
  // here).
  if (!M.rope_lds) load_tree_rope(TR, p.rope, M.pos_j, tid);  // uniform per wavefront
  TileRegs R0, R;
  load_ctx_tile(R0, G, c0, tid);
  load_ctx_tile(R, G, c0 + kTile, tid);
  if (M.rope_lds) read_tree_rope_lds(TR, smem + kRopeOff, M.pos_j - M.ctx, tid);
  const char* qbuf = smem;
  const char* tree_stage = smem + kStageBytes;
  store_tree_tile(smem + kStageBytes, smem, TR, t_real, p.scale * kLog2e, sp == 0, tid);
  lds_sync();
  u32x4 qv[kM];       // the lane's 8 dims of each query (rows >= t_real are zero)
  uint32_t anc_m[kM];  // ancestor-or-self bitmask of each query (nodes < 8: low word), uniform
  State st[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    qv[m] = *reinterpret_cast<const u32x4*>(qbuf + m * kQRow + 16 * dc);
    anc_m[m] = __builtin_amdgcn_readfirstlane((uint32_t)__shfl(anc, m));
    reset(st[m]);
  }
  // This lane group's tokens of tile t: c0 + 64 t + 16 pp + tid / 16.  Rows
  // past the split's end (the last page's tail, or a page re-read past the
  // end) are masked, and their values zeroed.
  const int tok_lane = c0 + (tid >> 4);
  auto consume = [&](const TileRegs& X, int t) {
    const int tok = tok_lane + kTile * t;
    u32x4 v[4];
    bool ok[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      ok[pp] = tok + 16 * pp < c1;
      v[pp] = ok[pp] ? X.v[pp] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      float s[4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const float d = group_sum(dot8(qv[m], X.k[pp], 0.f));
        s[pp] = ok[pp] ? d : -INFINITY;
      }
      add_tokens(st[m], s, v);
    }
  };
  // Tile 0 (R0) is consumed first; then the tiles alternate between R and a
  // second register tile, each refilled with the tile two ahead.
  TileRegs R2;
  if (n_tiles > 0) {
    load_ctx_tile(R2, G, c0 + 2 * kTile, tid);
    consume(R0, 0);
  }
  int t = 1;
#pragma unroll 1
  for (; t + 1 < n_tiles; t += 2) {
    const u32x4 ia = fetch_page_ids(G, c0 + kTile * (t + 2));
    const u32x4 ib = fetch_page_ids(G, c0 + kTile * (t + 3));
    consume(R, t);
    issue_ctx_tile(R, G, ia, c0 + kTile * (t + 2), tid);
    consume(R2, t + 1);
    issue_ctx_tile(R2, G, ib, c0 + kTile * (t + 3), tid);
  }
  if (t < n_tiles) consume(R, t);
  if (sp == 0 && wv < 2) {  // the tree keys, rotated as stored (zero rows past t_real)
    const int j = 4 * wv + grp;
    const u32x4 kk = *reinterpret_cast<const u32x4*>(tree_stage + j * kKRow + 16 * dc);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(tree_stage + kKBytes + j * kVRow + 16 * dc);
    const u32x4 v4[4] = {vv, vv, vv, vv};
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const float d = group_sum(dot8(qv[m], kk, 0.f));
      const float s4[4] = {(j < t_real && ((anc_m[m] >> j) & 1u)) ? d : -INFINITY, -INFINITY,
                           -INFINITY, -INFINITY};
      add_tokens(st[m], s4, v4);
    }
  }
  // Merge the 16 lane-group states of each query through LDS.
  __syncthreads();  // the query buffer and the tree tile are no longer read
  float* s_o = reinterpret_cast<float*>(smem);  // [16 states][kM][128]
  float* s_ml = s_o + 16 * kM * kD;             // [16 states][kM][2]
  const int si = tid >> 4;
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    float* o = s_o + (si * kM + m) * kD + 8 * dc;
    *reinterpret_cast<f32x4*>(o) = f32x4{st[m].o[0], st[m].o[1], st[m].o[2], st[m].o[3]};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{st[m].o[4], st[m].o[5], st[m].o[6], st[m].o[7]};
    if (dc == 0) {
      s_ml[(si * kM + m) * 2] = st[m].m;
      s_ml[(si * kM + m) * 2 + 1] = st[m].l;
    }
  }
  __syncthreads();
  const int bh = b * p.H + h;
  for (int idx = tid; idx < kM * (kD / 4); idx += kThreads) {
    const int m = idx / (kD / 4), d4 = 4 * (idx % (kD / 4));
    if (m >= t_real) continue;
    float M = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) M = fmaxf(M, s_ml[(s2 * kM + m) * 2]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      const float w = __builtin_amdgcn_exp2f(s_ml[(s2 * kM + m) * 2] - Mu);  // -inf -> 0
      L += w * s_ml[(s2 * kM + m) * 2 + 1];
      o += w * *reinterpret_cast<const f32x4*>(s_o + (s2 * kM + m) * kD + d4);
    }
    if (nsplit == 1) {
      const float inv = L > 0.f ? 1.0f / L : 0.f;
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + (((size_t)b * T + m) * p.H + h) * kD +
                                d4) = __builtin_bit_cast(u32x2, __builtin_convertvector(o * inv, bf16x4));
    } else {
      const size_t row = ((size_t)bh * p.splits + sp) * T + m;
      *reinterpret_cast<f32x4*>(p.ws_o + row * kD + d4) = o;
      if (d4 == 0) p.ws_ml[row] = float2{M, L};
    }
  }
  if (nsplit == 1) {  // padding rows (and rows past the real ones) are zeros
    for (int idx = tid; idx < (T - t_real) * 16; idx += kThreads) {
      const int m = t_real + (idx >> 4), ch = idx & 15;
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + (((size_t)b * T + m) * p.H + h) * kD +
                                8 * ch) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}


// ---- Round trip 1: ctx_len, page ids, tree rows, then the q rows and the
// tree k/v rows.  Every load is unconditional (row indices clamped into
// their arrays, values masked where they are used), so the wavefront issues
// them back to back; the page ids go to s_pages (visible after the caller's
// next LDS barrier, which waits for them and the tree rows alone: the q and
// tree k/v rows stay in flight into round trip 2).  Returns false (uniform)
// when the split lies beyond the context.
__device__ __forceinline__ bool item_round_trip1(const VerifyParams& p, int b, int h, int hk,
                                                 int sp, int c0, int ctx0, char* rope_lds,
                                                 int* s_pages, TreeRaw& TR, ItemMeta& M,
                                                 int tid) {
  const int lane = tid & 63;
  const int T = p.T;
  const int ctx_raw = p.ctx_lens[b];
  // c0 < max(max_ctx, 1) <= 16 * max_blocks for every split of the plan, so
  // max_pages >= 1 and the clamped page index stays inside the table row.
  const int32_t* table_row = p.block_table + (size_t)b * p.max_blocks + (c0 >> 4);
  const int max_pages = min(p.chunk / kPage, p.max_blocks - (c0 >> 4));
  static_assert(kMaxSplitPages <= 2 * kThreads, "two page ids per thread");
  const int blk_raw0 = table_row[min(tid, max_pages - 1)];
  const int blk_raw1 = table_row[min(tid + kThreads, max_pages - 1)];
  const int row_l = min(lane, T - 1);
  const int par_raw = p.tree_parent[(size_t)b * T + row_l];
  const int dep_raw = p.tree_depth[(size_t)b * T + row_l];
  // The (cos, sin) rows ctx0 .. ctx0 + kRopeRows - 1, 16 bytes per thread
  // (ctx0 < 0, ctx_len not known at launch: rows from 0, not used).
  static_assert(kRopeRows * kRopeRowBytes == 16 * kThreads, "one chunk per thread");
  const int rope_row = min(max(ctx0, 0) + (tid >> 5), p.rope_max_pos - 1);
  const u32x4 rope_chunk =
      *reinterpret_cast<const u32x4*>(p.rope + (size_t)rope_row * kD + 4 * (tid & 31));
  // Every split rotates its queries; only split 0 uses the tree k/v rows (the
  // others read row 0 over and over).
  load_tree_raw(TR, p, b, h, hk, sp == 0 ? T - 1 : 0, tid);

  M.ctx = clampi(ctx_raw, 0, p.max_ctx);
  M.nsplit = M.ctx == 0 ? 1 : (M.ctx + p.chunk - 1) / p.chunk;
  if (sp >= M.nsplit) return false;
  M.c1 = min(M.ctx, c0 + p.chunk);
  M.npages = (M.c1 - c0 + kPage - 1) / kPage;  // <= max_pages
  // Entry 0 is written even for an empty split: the first two tiles load
  // unconditionally.
  if (tid < max(M.npages, 1))
    s_pages[tid] = (tid < M.npages && blk_raw0 >= 0 && blk_raw0 < p.num_blocks) ? blk_raw0 : 0;
  if (tid + kThreads < M.npages)
    s_pages[tid + kThreads] = (blk_raw1 >= 0 && blk_raw1 < p.num_blocks) ? blk_raw1 : 0;
  *reinterpret_cast<u32x4*>(rope_lds + 16 * tid) = rope_chunk;
  const int par = lane < T ? par_raw : kPadParent;
  M.dep = lane < T ? dep_raw : 0;

  const bool real = lane < T && par != kPadParent;
  const uint64_t real_mask = __ballot(real);
  M.t_real = real_mask == ~0ull ? 64 : __builtin_ctzll(~real_mask);  // real prefix
  const bool linked = lane < M.t_real && (lane == 0 ? par == -1 : (par >= 0 && par < lane));
  uint64_t anc = linked ? (1ull << lane) : 0ull;
  int up = (linked && lane > 0) ? par : lane;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const uint64_t a_up = __shfl(anc, up);
    const int up_up = __shfl(up, up);
    anc |= a_up;
    up = up_up;
  }
  M.anc = anc;
  const int dj = clampi(__shfl(M.dep, tid >> 2), 0, T - 1);
  M.pos_j = M.ctx + dj;
  M.rope_lds = ctx0 == M.ctx && __ballot((tid >> 2) < M.t_real && dj >= kRopeRows) == 0ull;
  return true;
}

// A work item whose tree has at most kSmallTree real nodes: round trip 1 as
// on the matrix-core path, then the vector-ALU path above.
__device__ __forceinline__ void small_tree_workgroup(const VerifyParams& p, int b, int h, int sp,
                                                     int ctx0, char* smem, int* s_pages,
                                                     int tid) {
  const int hk = h / (p.H / p.Hkv);
  const int c0 = sp * p.chunk;
  TreeRaw TR;
  ItemMeta M;
  if (!item_round_trip1(p, b, h, hk, sp, c0, ctx0, smem + kRopeOff, s_pages, TR, M, tid))
    return;  // uniform
  lds_sync();  // s_pages visible
  const Geo G{static_cast<const uint16_t*>(p.kv_pages), s_pages, c0, hk, p.Hkv,
              max(M.npages - 1, 0)};
  const int n_tiles = (M.c1 - c0 + kTile - 1) / kTile;
  if (M.t_real <= 1)
    small_tree_item<1>(p, G, TR, M, smem, n_tiles, c0, b, h, sp, tid);
  else
    small_tree_item<2>(p, G, TR, M, smem, n_tiles, c0, b, h, sp, tid);
}

// Launch slot -> (sequence, head, split).  A (sequence, split) group holds H
// work items of the same length (the split's tokens).  With at most 64
// groups, the groups that exist are ranked by length (longest first, equal
// lengths in (sequence, split) order) and each group's heads take
// consecutive slots; slots past the real items leave at once.  When there are
// between one and two items per CU, slots 0..n_cu-1 take the longest items
// and slot n_cu + i takes the i-th shortest: the dispatcher fills every CU
// with slots i and i + n_cu, so each CU then holds one long and one short item
// and about the average number of tiles.  With more items than that,
// longest-first order lets the dispatcher hand the short tail to whichever CU
// frees up first.  With more than 64 groups the order is (sequence, head)
// major, split minor.  Every lane of the wavefront takes part (lane = group).
//
// Grouped query heads: the workgroups that share a KV head stream the same
// pages, and they meet in an L2 only on the same XCD.  Workgroup s runs on
// XCD s mod 8, and the heads of one group (one sequence and split) take
// consecutive slots from a multiple of 8 on (H a multiple of 8), so head
// offset o lands on XCD o mod 8 (or 7 - o mod 8 for the short half, whose
// slots run backwards).  With fewer KV heads than query heads, offset o
// takes head (o mod 8) * H/8 + o / 8: each XCD gets H/8 consecutive heads,
// that is whole groups of H/Hkv heads sharing a KV head (or, with more than
// H/8 heads per KV head, an eighth of the XCDs per KV head).  On the 7B
// batch-16 shape with 8 or 4 KV heads this cut the launch from 58-61 to
// 42-43 us; with one KV head per query head the order is unchanged.
__device__ __forceinline__ int grouped_head(const VerifyParams& p, int o) {
  return (p.Hkv < p.H && (p.H & 7) == 0) ? (o & 7) * (p.H >> 3) + (o >> 3) : o;
}

__device__ __forceinline__ bool launch_item(const VerifyParams& p, int slot, int lane, int& b,
                                            int& h, int& sp, bool& small, int& ctx0, bool& eager) {
  const int G = p.B * p.splits;
  small = false;
  ctx0 = -1;
  {
    const int n_grid = p.B * p.H * p.splits;
    eager = !(n_grid > p.n_cu && n_grid < 2 * p.n_cu);
  }
  if (G > 64 || p.n_cu <= 0) {
    b = (slot / p.splits) / p.H;
    h = (slot / p.splits) % p.H;
    sp = slot % p.splits;
    if (p.splits == 1) h = grouped_head(p, h);  // slot mod 8 = h mod 8
    return true;
  }
  int len = -1;  // tokens of the group's split; -1: the split does not exist
  int small_l = 0;  // the group's tree has at most kSmallTree real nodes
  int ctx_l = 0;    // the group's ctx_len (clamped)
  if (lane < G) {
    const int j = lane / p.splits, s = lane - j * p.splits;
    const int ctx_raw = p.ctx_lens[j];
    const int par_cut = p.tree_parent[(size_t)j * p.T + min(kSmallTree, p.T - 1)];
    const int c = clampi(ctx_raw, 0, p.max_ctx);
    ctx_l = c;
    const int n = c == 0 ? 1 : (c + p.chunk - 1) / p.chunk;
    if (s < n) len = min(p.chunk, c - s * p.chunk);
    // Real nodes form a prefix, so a padding node at index kSmallTree (or a
    // tree of at most kSmallTree rows) bounds the real ones by kSmallTree.
    small_l = p.T <= kSmallTree || par_cut == kPadParent;
  }
  const int N = __popcll(__ballot(len >= 0)) * p.H;
  if (slot >= N) return false;  // uniform
  // `eager`: the tile loop issues a tile's loads before the barrier that
  // follows the previous tile's store, not after it; except when some CUs
  // hold two items and others one, where that measured slower (13B-shaped
  // batch 8: +6.5 us, against batch 16 -0.2 to -0.6 us, stress -3.5 us,
  // batch 1 -0.1 us).  Without the ranking the same rule takes the grid size.
  eager = !(N > p.n_cu && N < 2 * p.n_cu);
  int r = slot;
  if (N > p.n_cu && N <= 2 * p.n_cu && slot >= p.n_cu) r = N - 1 - (slot - p.n_cu);
  // Each lane counts the groups ranked above its own; group j's length is
  // read from lane j with a lane read (a lane shuffle would take a round
  // trip through the LDS crossbar per group).
  int rank = 0;
  for (int j = 0; j < G; ++j) {  // uniform
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len) || (lj == len && j < lane);
  }
  const int gr = r / p.H;
  h = grouped_head(p, r - gr * p.H);
  const uint64_t hit = __ballot(lane < G && rank == gr);
  const int grp = hit ? __builtin_ctzll(hit) : 0;
  b = grp / p.splits;
  sp = grp - b * p.splits;
  small = __builtin_amdgcn_readlane(small_l, grp) != 0;
  ctx0 = __builtin_amdgcn_readlane(ctx_l, grp);
  return true;
}


__global__ __launch_bounds__(kThreads, TA_WG_PER_CU) void verify_mfma_kernel(VerifyParams p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  static_assert(4 * kHalfPark * sizeof(float) <= 2 * kStageBytes, "merge area");
  __shared__ __attribute__((aligned(16))) int s_pages[kMaxSplitPages];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int qt = wv >> 1, th = wv & 1;
  const int g = lane >> 5, r32 = lane & 31;
  int b, h, sp;
  bool small;
  int ctx0;  // ctx_len read by the launch ranking (-1: not read)
  bool eager;
  if (!launch_item(p, blockIdx.x, lane, b, h, sp, small, ctx0, eager)) return;
  static_assert(kRopeOff + kRopeRows * kRopeRowBytes <= kStageBytes, "rope rows in stage 0");
  if (small) {  // uniform: a tree of at most kSmallTree real nodes
    small_tree_workgroup(p, b, h, sp, ctx0, smem, s_pages, tid);
    return;
  }
  const int bh = b * p.H + h;
  const int hk = h / (p.H / p.Hkv);
  const int T = p.T;
  const int q = 32 * qt + r32;
  const int c0 = sp * p.chunk;

  TreeRaw TR;
  ItemMeta M;
  if (!item_round_trip1(p, b, h, hk, sp, c0, ctx0, smem + kRopeOff, s_pages, TR, M, tid))
    return;  // uniform
  const int ctx = M.ctx, nsplit = M.nsplit, c1 = M.c1, npages = M.npages, t_real = M.t_real;
  const uint64_t anc = M.anc;
  const int pos_j = M.pos_j;
  const int nqt = t_real > 32 ? 2 : 1;
  const bool active = qt < nqt;
  const uint64_t anc_q = __shfl(anc, q);
  const bool row_real = active && q < t_real;

  lds_sync();  // s_pages visible; the q and tree k/v rows may still be in flight
  // ---- round trip 2: the (cos, sin) rows and context tiles 0 and 1; the
  // queries are rotated and the tree tile is built and computed while the
  // tiles load.
  Geo G{static_cast<const uint16_t*>(p.kv_pages), s_pages, c0, hk, p.Hkv, max(npages - 1, 0)};
  const int n_tiles = (c1 - c0 + kTile - 1) / kTile;
  // Node tid/4's (cos, sin) row, for its key and its query: from LDS, or
  // (deep trees) from the table before the tiles are issued.
  if (!M.rope_lds) load_tree_rope(TR, p.rope, pos_j, tid);  // uniform per wavefront
  TileRegs R0;  // context tile 0
  TileRegs R;   // context tile t + 1 while tile t is computed
  load_ctx_tile(R0, G, c0, tid);  // unconditional: the compiler counts the loads
  load_ctx_tile(R, G, c0 + kTile, tid);
  if (M.rope_lds) read_tree_rope_lds(TR, smem + kRopeOff, pos_j - ctx, tid);

  char* stage0 = smem;
  char* stage1 = smem + kStageBytes;
  // While context tiles 0 and 1 load, the rotated queries go to a stage that
  // is free until a tile is stored there: split 0 puts its tree tile in
  // stage 1 and its queries in stage 0 (one more barrier before tile 0 takes
  // stage 0); the other splits put their queries in stage 1, which tile 1
  // only takes after the barrier that follows tile 0's store.
  static_assert(kTile * kQRow <= kStageBytes, "query buffer in a stage");
  char* qbuf = sp == 0 ? stage0 : stage1;
  store_tree_tile(stage1, qbuf, TR, t_real, p.scale * kLog2e, sp == 0, tid);
  lds_sync();
  WaveState st;
  reset(st);
  const LaneOffs L = lane_offsets(lane, th, kKBytes);
  u32x4 qf[8];
  load_q_frags(qf, qbuf, q, g);
  if (sp == 0) {  // uniform
    if (active) compute_tile<kTreeTile>(st, qf, stage1, L, kTile, anc_q);
    lds_sync();  // query buffer read by every wavefront: stage 0 takes tile 0
  }
  auto rows_of = [&](int t) { return min(kTile, c1 - (c0 + kTile * t)); };
  if (n_tiles > 0) store_tile(R0, stage0, rows_of(0), tid);
  lds_sync();  // stage 0 filled; stage 1's tree or query reads done; tile 1 stays in flight
  if (n_tiles > 0) {
    // Every tile but the last is full: one straight-line path, no masking.
    // The page ids of tile t + 2 are read from LDS before tile t is computed.
    for (int t = 0; t < n_tiles - 1; ++t) {
      char* cur = (t & 1) ? stage1 : stage0;
      char* nxt = (t & 1) ? stage0 : stage1;
      const u32x4 ids = fetch_page_ids(G, c0 + kTile * (t + 2));
      if (active) compute_tile<kFull>(st, qf, cur, L, kTile, 0ull);
      store_tile(R, nxt, rows_of(t + 1), tid);
      // R is free once stored: the next loads go out before or after the
      // barrier (an LDS-only barrier, so loads in flight stay in flight).
      if (eager && t + 2 < n_tiles) issue_ctx_tile(R, G, ids, c0 + kTile * (t + 2), tid);
      lds_sync();
      if (!eager && t + 2 < n_tiles) issue_ctx_tile(R, G, ids, c0 + kTile * (t + 2), tid);
    }
    // The last tile may end mid-tile.
    const int t = n_tiles - 1;
    char* cur = (t & 1) ? stage1 : stage0;
    const int n_valid = c1 - (c0 + kTile * t);
    if (active) {
      if (n_valid >= kTile)
        compute_tile<kFull>(st, qf, cur, L, kTile, 0ull);
      else
        compute_tile<kPartial>(st, qf, cur, L, n_valid, 0ull);
    }
  }

  // Merge the two token halves of each query tile; each wavefront of the
  // pair finishes two of the four d-tiles.  The halves are parked in the
  // stage that the last tile did not use (every wavefront passed a barrier
  // after its last read of it), so no barrier comes first; the output tile
  // then takes the last tile's stage, free after the barrier that follows
  // the parking.
  char* last_stage = (n_tiles == 0 || ((n_tiles - 1) & 1)) ? stage1 : stage0;
  char* free_stage = last_stage == stage0 ? stage1 : stage0;
  static_assert(4 * kHalfPark * sizeof(float) <= kStageBytes, "park area in a stage");
  static_assert(kTile * kOutRow <= kStageBytes, "output tile in a stage");
  // (th is uniform over a wavefront: each branch indexes the accumulators
  // with constants.)
  float* park = reinterpret_cast<float*>(free_stage);
  if (active) {
    if (th == 0)
      park_half<2>(st, park + (2 * qt) * kHalfPark, lane);
    else
      park_half<0>(st, park + (2 * qt + 1) * kHalfPark, lane);
  }
  __syncthreads();
  if (active) {
    if (th == 0)
      merge_half<0>(st, park + (2 * qt + 1) * kHalfPark, lane);
    else
      merge_half<1>(st, park + (2 * qt) * kHalfPark, lane);
    st.l = sum_xor32(st.l);
  }
  if (nsplit == 1) {  // uniform
    char* tile = last_stage;
    if (th == 0)
      stage_out<0>(st, tile, q, row_real, g);
    else
      stage_out<2>(st, tile, q, row_real, g);
    __syncthreads();
    store_out(tile, p, b, h, tid);
  } else if (th == 0) {
    write_partial_half<0>(st, p, bh, sp, q, T, row_real, g, true);
  } else {
    write_partial_half<2>(st, p, bh, sp, q, T, row_real, g, false);
  }
}

// Merge the (m, l, O) partials of every (sequence, head) whose context took
// more than one split, and write its `out` rows (padding rows as zeros).
// One workgroup per 16 rows of a (sequence, head), so that a small batch
// still spreads the partial reads over many CUs.  A separate launch: the
// kernel boundary makes every split's partials visible, where a device-wide
// fence inside the verify kernel would write back and invalidate the L2 of
// its XCD once per workgroup.
constexpr int kCombineRows = 16;  // rows of one (sequence, head) per combine workgroup
__global__ __launch_bounds__(kThreads) void combine_kernel(VerifyParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int T = p.T;
  // ctx_len and the tree rows in one round trip (the row index is clamped
  // into the array and masked below).
  const int ctx_raw = p.ctx_lens[b];
  const int par_raw = p.tree_parent[(size_t)b * T + min(lane, T - 1)];
  const int ctx = clampi(ctx_raw, 0, p.max_ctx);
  const int nsplit = ctx == 0 ? 1 : (ctx + p.chunk - 1) / p.chunk;
  if (nsplit == 1) return;
  const int par = lane < T ? par_raw : kPadParent;
  const uint64_t real_mask = __ballot(lane < T && par != kPadParent);
  const int t_real = real_mask == ~0ull ? 64 : __builtin_ctzll(~real_mask);
  // Thread: row cq of this workgroup's 16, dims 8 ch .. 8 ch + 7.
  const int cq = kCombineRows * blockIdx.y + (tid >> 4), ch = tid & 15;
  if (cq >= T) return;
  uint16_t* orow = static_cast<uint16_t*>(p.out) + (((size_t)b * T + cq) * p.H + h) * kD + 8 * ch;
  f32x8 acc = {};
  float L = 0.f;
  if (cq < t_real) {
    // Splits are read in unrolled groups of four whose loads are all issued
    // before any is used (one memory round trip per group, not per split),
    // and merged online: the running max moves to the group's max and the
    // sums so far are rescaled.  An index past the last split reads the last
    // one again and is given no weight.
    const size_t row0 = (size_t)bh * p.splits * T + cq;
    auto row_of = [&](int s) { return row0 + (size_t)min(s, nsplit - 1) * T; };
    float M = -INFINITY;
    for (int s0 = 0; s0 < nsplit; s0 += 4) {
      float2 ml[4];
      f32x8 o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t row = row_of(s0 + u);
        ml[u] = p.ws_ml[row];
        o[u] = reinterpret_cast<const f32x8*>(p.ws_o + row * kD)[ch];
      }
      __builtin_amdgcn_sched_barrier(0);  // the group's loads all go out first
      float Mn = M;
#pragma unroll
      for (int u = 0; u < 4; ++u) Mn = fmaxf(Mn, ml[u].x);  // a repeated split leaves it as is
      const float Mu = Mn == -INFINITY ? 0.f : Mn;
      const float f = __builtin_amdgcn_exp2f(M - Mu);  // 0 while nothing has been added
      L *= f;
      acc *= f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = s0 + u < nsplit ? __builtin_amdgcn_exp2f(ml[u].x - Mu) : 0.f;
        L += w * ml[u].y;
        acc += w * o[u];
      }
      M = Mn;
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  *reinterpret_cast<u32x4*>(orow) = __builtin_bit_cast(u32x4, __builtin_convertvector(acc * inv, bf16x8));
}

}  // namespace


hipError_t launch_verify_mfma(const VerifyParams& p, hipStream_t stream) {
  const long long grid = (long long)p.B * p.H * p.splits;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(verify_mfma_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_split_combine(const VerifyParams& p, hipStream_t stream) {
  static_assert(kThreads == 16 * kCombineRows, "16 threads per row");
  const unsigned row_groups = (unsigned)((p.T + kCombineRows - 1) / kCombineRows);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(p.B * p.H), row_groups), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace ta
