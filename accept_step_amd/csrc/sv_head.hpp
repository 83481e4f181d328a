// sv_head.hpp -- the k-split streaming product and the fused verify kernel (gfx950).
//
// Same contraction as sv_gemm.hpp, out[m, v] = sum_k X[m, k] W[v, k] with W streamed
// once from HBM, but with each load instruction covering whole 128-byte lines: HBM
// reads with non-temporal loads reach about 7.2 TB/s on MI355X when every row
// segment a wavefront touches is at least 128 contiguous bytes, against about 6.4
// TB/s for the 64-byte row segments that the plain 16x16x32 operand layout gives.
//
// k-split virtual rows.  v_mfma_f32_16x16x32_bf16 multiplies a 16 x 32 operand A by
// a 32 x 16 operand B.  Here the 16 rows of A are TR = 16 / S rows of W, each split
// into S interleaved parts of its k range: virtual row r = (W row r / S, part r % S).
// The 16 columns of B are likewise CPB = 16 / S rows of X times the same S parts.
// Output entry (r, c) is a partial dot product when the parts of r and c agree and
// meaningless otherwise; summing the S partials of a (W row, X row) pair over the
// S lanes that hold them gives the product.  Lane (r, g) of step j reads 16-byte
// piece 4S*j + S*g + r % S of W row r / S, so the 4S lanes of a W row read 64*S
// contiguous bytes.  The matrix cores do S times more work per byte than needed,
// which leaves them far from busy at these shapes (a few rows of X).
//
// The products of a workgroup's tiles are kept in LDS.  After the stream, the
// workgroup writes them out if asked, reduces its share of every row to a
// statistics partial (max, sum of exp((l - max)/T), lowest-index argmax), and
// records the draft-token logits it owns.  Then, depending on the mode:
//   HEAD_PRODUCT  nothing more (decoder projections, verify_forward);
//   HEAD_ACCEPT   the last workgroup to finish applies the rule (greedy, or the
//                 acceptance half of sampling);
//   HEAD_SAMPLE   the whole sampling rule in one launch: after a grid barrier every
//                 workgroup merges the partials and decides n for every sequence
//                 (same inputs, same arithmetic, same result), draws the Gumbel-max
//                 of row n over its own slice of the vocabulary straight from LDS,
//                 and stores its slice winner; the last workgroup through merges the
//                 winners and commits.  The barrier needs every workgroup resident at
//                 once (the host checks the occupancy); its wait is bounded, and a
//                 timed-out wait marks the step's outputs invalid instead of hanging.
// The row statistics are folded tile by tile in the product's epilogue, where they
// overlap the loads in flight.  Counts between workgroups are two-level (one counter
// per XCD on its own cache line, then one at the top): hundreds of workgroups
// incrementing one line at the same moment serialise for tens of microseconds.
// Rule and sampler: [MTP-deep-dive] 2.2, [Infra-ch8] "why the output does not
// change", [Self-spec] 3.1-3.3; see sv_accept.hpp.
#pragma once

#include "sv_accept.hpp"
#include "sv_device.hpp"
#include "sv_gemm.hpp"

namespace sv {

constexpr int HEAD_WAVES = 4;      // wavefronts per workgroup
constexpr int HEAD_MAX_ROWS = 24;  // most rows of X (M) the k-split kernel takes
constexpr int HEAD_PRODUCT = 0, HEAD_ACCEPT = 1, HEAD_SAMPLE = 2;
constexpr unsigned HEAD_SPIN_LIMIT = 1u << 20;   // default polls of the barrier count (about a second)

// The counter block at the start of the workspace (zero between launches), in
// 32-bit words.  Line 0: the top counts and a sticky error flag; lines 1-8: per-group
// arrival counts; lines 9-16: per-group finishing counts.
constexpr int CNT_BYTES = 4096;
constexpr int CNT_LINE = 32;                      // words per 128-byte line
constexpr int CNT_GROUPS = 8;                     // workgroups are dispatched round-robin over 8 XCDs
constexpr int CNT_TOP_ARRIVE = 0, CNT_TOP_DONE = 1, CNT_ERROR = 2;
constexpr int CNT_GRP_ARRIVE = 1 * CNT_LINE, CNT_GRP_DONE = 9 * CNT_LINE;
// The fused sampler hands data between workgroups as epoch-tagged 64-bit words (value
// bits low, launch epoch high) and needs no counter: readers poll until every word they
// need carries the current epoch.  The epoch lives in the counter block: each launch
// uses the stored value plus one and its finishing workgroup stores it once every
// workgroup is known to have read it.  POISON marks a workspace on which some workgroup
// had not run when the step gave up (see HEAD_SAMPLE below).
constexpr int CNT_EPOCH = 17 * CNT_LINE, CNT_FAIL = 18 * CNT_LINE;
constexpr unsigned EPOCH_POISON = 0xffffffffu;

struct HeadArgs {
  const bf16_t* W[MAX_SEG];   // [N_s, K] row-major
  float* out[MAX_SEG];        // [M, N_s] row-major (written when write_out)
  int N[MAX_SEG];
  int tile_end[MAX_SEG];      // cumulative TR-row tile counts
  int nseg;
  const bf16_t* X;            // [M, K]
  int M, K;
  int gpt;                    // work items per tile (K / (32 * S * GRP))
  int nloc;                   // LDS products kept per X row: tiles per workgroup * TR
  int write_out;
  int mode;
  // statistics and rule (single segment)
  RowPart* part;              // [gridDim.x, M]; null: no statistics
  float c_stat;               // log2(e) / T; 0 = max / argmax only
  float* xlogit;              // [M] draft-token logits (rule modes)
  unsigned* counter;          // the counter block
  AcceptArgs acc;             // acc.P == gridDim.x
  SamplePart* spart;          // unused by the k-split kernel
  // HEAD_SAMPLE hand-off records, 4 tagged words each: statistics partials [grid][M],
  // group partials [8][M], draft logits [M] (1 word each), slice winners [B][grid]
  unsigned long long* recs;
  int rec_grid;               // grid the record regions are sized for
  unsigned spin_limit;        // polls of the barrier count before giving up
  // decoder fusions (product mode)
  const float* Xf;            // non-null: X = bf16(Xf * rsqrt(mean(Xf^2) + eps) * norm_w) per row, Xf [M, K]
  const bf16_t* norm_w;       // [K]
  const float* ss_in;         // [ss_parts, M] partial sums of squares of the Xf rows
  int ss_parts;
  float eps;
  int residual;               // the products are added into out (out[m, n] += ...)
  float* ss_out;              // residual: [gridDim.x, M] sums of squares of the updated rows per workgroup
  // write_out == 2: SwiGLU pairing (two segments of equal N, gate then up): the wavefront
  // that streams gate tile t streams up tile t right after it, and the epilogue writes
  // hout[m, n] = bf16(SiLU(gate) * up) instead of the two products
  bf16_t* hout;               // [M, N_0]
};
// Launches cost more once the explicit arguments pass 368 bytes (+0.2-0.3 us each
// measured at 376: the MTP draft round 758 -> 775 us, the full-model step +0.03 ms).
static_assert(sizeof(HeadArgs) <= 368, "k_head's arguments past the cheap launch size");

// Bytes of dynamic LDS: the M rows of X plus one zero row that the lanes of padding
// rows (past M in the last column block) read, each row padded by 16*S bytes so the
// lanes of a k-group hit distinct banks; then the kept products.  Kp is K rounded up
// to whole work items (zeros past K: see k_head).
__host__ __device__ inline size_t head_lds_x(int M, int Kp, int S) {
  return (size_t(M + 1) * (Kp + 8 * S) * 2 + 15) / 16 * 16;
}
__host__ __device__ inline size_t head_lds(int M, int Kp, int S, int nloc) {
  return head_lds_x(M, Kp, S) + size_t(M) * nloc * 4;
}

__device__ __forceinline__ TileRef head_tile(const HeadArgs& a, int tile, int TR) {
  const int seg = (a.nseg > 1 && tile >= a.tile_end[0]) ? ((a.nseg > 2 && tile >= a.tile_end[1]) ? 2 : 1) : 0;
  TileRef t;
  t.W = pick(seg, a.W[0], a.W[1], a.W[2]);
  t.out = pick(seg, a.out[0], a.out[1], a.out[2]);
  t.N = pick(seg, a.N[0], a.N[1], a.N[2]);
  t.v0 = (tile - pick(seg, 0, a.tile_end[0], a.tile_end[1])) * TR;
  return t;
}

// Paired tiles.  Wavefront ``first`` (= workgroup * HEAD_WAVES + wave) takes the gate
// and the up tile of rows u * span + slot, u = 0, 1, ..., with slot = wave * grid +
// workgroup: numbered wavefront-major, the last partial round spreads over all
// workgroups before any takes two (workgroup-major, the first workgroups would each take
// four while the rest idle).  Its rounds 2u and 2u + 1 are that gate and up tile.
__device__ __forceinline__ int head_pair_slot(int first, int grid) {
  return (first % HEAD_WAVES) * grid + first / HEAD_WAVES;
}
// Tile ``tile`` = round * span + first (span = grid * HEAD_WAVES) of a paired product.
__device__ __forceinline__ TileRef head_tile_pair(const HeadArgs& a, int tile, int TR) {
  const int span = int(gridDim.x) * HEAD_WAVES, i = tile / span, f = tile - i * span;
  TileRef t;
  t.W = (i & 1) ? a.W[1] : a.W[0];
  t.out = (i & 1) ? a.out[1] : a.out[0];
  t.N = a.N[0];
  t.v0 = ((i >> 1) * span + head_pair_slot(f, gridDim.x)) * TR;
  return t;
}

// Tiles of the wavefront whose first tile is ``first``: paired, two for each gate tile
// slot, slot + span, ... below the segment's tile count.
__device__ __forceinline__ int head_tiles_of(const HeadArgs& a, int first, int span, int ntiles, bool pair) {
  if (pair) {
    const int P = a.tile_end[0], slot = head_pair_slot(first, span / HEAD_WAVES);
    return slot < P ? 2 * ((P - 1 - slot) / span + 1) : 0;
  }
  return first < ntiles ? (ntiles - 1 - first) / span + 1 : 0;
}

// Global tile of local tile ``lt`` of workgroup ``wg``: wavefront lt % 4, its (lt / 4)-th tile.
__device__ __forceinline__ int head_global_tile(int wg, int lt, int grid) {
  return wg * HEAD_WAVES + (lt % HEAD_WAVES) + (lt / HEAD_WAVES) * grid * HEAD_WAVES;
}

// Weights are read through buffer descriptors (one per segment, bounded to the
// segment's bytes): 32-bit offsets from a scalar base leave less vector address work
// per load than 64-bit global addresses (805 MB streamed in 109 us against 112 us),
// and reads past the segment's end return zeros, so the rows beyond N of a ragged last
// tile need no clamping (their products are discarded).
struct HeadItem {
  __amdgpu_buffer_rsrc_t rs;
  unsigned soff;              // byte offset of the item within its segment (uniform)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const bf16_t* W, int N, int K) {
  // The tile (hence the segment) is uniform over the wavefront; saying so keeps the
  // descriptor in scalar registers (otherwise every load becomes a loop over lanes).
  const uint64_t wp = reinterpret_cast<uint64_t>(W);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(wp)), hi = __builtin_amdgcn_readfirstlane(uint32_t(wp >> 32));
  void* base = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  const int bytes = __builtin_amdgcn_readfirstlane(int(unsigned(N) * unsigned(K) * 2u));
  // raw buffer, no stride; num_records = the segment's bytes (below 4 GB, checked on the host)
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, bytes, 0x00020000);
}

// Work item k of a wavefront whose tiles are first, first + tstride, ...: the segment's
// descriptor and the item's offset.  The lane adds (r / S) * K * 2 + its piece offset.
// Work item k of the wavefront whose tiles are round * tstride + slot (round = i >> psh
// for its i-th tile): plain (psh = 0, slot = first), tile i is round i over all segments;
// paired (psh = 1, slot = head_pair_slot), tiles 2u and 2u + 1 are the gate and the up
// tile of round u.  Selects only: a branch inside the stream loop makes the compiler keep
// fewer loads in flight across it (every product measured 15-25 % slower).
template <int S, bool PAIRABLE>
__device__ __forceinline__ HeadItem head_item(const HeadArgs& a, int k, int slot, int psh, int tstride, int item_k) {
  const int i = k / a.gpt, gg = k - i * a.gpt;
  if constexpr (!PAIRABLE) {
    const TileRef tr = head_tile(a, slot + i * tstride, 16 / S);
    HeadItem it;
    it.rs = head_rsrc(tr.W, tr.N, a.K);
    it.soff = __builtin_amdgcn_readfirstlane((unsigned(tr.v0) * unsigned(a.K) + unsigned(gg * item_k)) * 2u);
    return it;
  }
  const int tile = (i >> psh) * tstride + slot;
  const int segn = (a.nseg > 1 && tile >= a.tile_end[0]) ? ((a.nseg > 2 && tile >= a.tile_end[1]) ? 2 : 1) : 0;
  const int seg = psh ? (i & 1) : segn;
  const int t0 = tile - (psh ? 0 : pick(segn, 0, a.tile_end[0], a.tile_end[1]));
  HeadItem it;
  it.rs = head_rsrc(pick(seg, a.W[0], a.W[1], a.W[2]), pick(seg, a.N[0], a.N[1], a.N[2]), a.K);
  it.soff = __builtin_amdgcn_readfirstlane((unsigned(t0 * (16 / S)) * unsigned(a.K) + unsigned(gg * item_k)) * 2u);
  return it;
}

// Loads of one work item (non-temporal: each byte is used once).  The scheduling
// barrier keeps them issued ahead of the previous item's matrix work (the scheduler
// would otherwise sink them below it and halve the loads in flight).
template <int S, int NB, int GRP>
__device__ __forceinline__ void head_load(const HeadItem& it, unsigned voff, u32x4 (&buf)[GRP]) {
#pragma unroll
  for (int u = 0; u < GRP; ++u)
    buf[u] = __builtin_amdgcn_raw_buffer_load_b128(it.rs, voff + 64u * S * u, it.soff, 2 /* nt */);
  __builtin_amdgcn_sched_barrier(0);
}

// One work item: GRP steps of NB MFMAs.  The X operands of the item are read from
// LDS in one batch (lanes of padding rows read the zero row, so no read is conditional).
// A wavefront's first two work items, requested by the staging code once its own first
// loads are out.  Both are always requested (from the last tile, or item 0 again, when
// the wavefront has fewer; those registers are never used), so no branch hides them from
// the compiler's count of outstanding loads.
struct HeadFirst {
  int items, slot, psh, tstride, item_k, ntiles;
  unsigned voff;
};

template <int S, int NB, int GRP, bool PAIRABLE>
__device__ __forceinline__ void head_first_loads(const HeadArgs& a, const HeadFirst& hf, u32x4 (&bufA)[GRP],
                                                 u32x4 (&bufB)[GRP]) {
  const int f = min(hf.slot, (hf.psh ? a.tile_end[0] : hf.ntiles) - 1), k1 = hf.items > 1 ? 1 : 0;
  head_load<S, NB, GRP>(head_item<S, PAIRABLE>(a, 0, f, hf.psh, hf.tstride, hf.item_k), hf.voff, bufA);
  head_load<S, NB, GRP>(head_item<S, PAIRABLE>(a, k1, f, hf.psh, hf.tstride, hf.item_k), hf.voff, bufB);
}

template <int S, int NB, int GRP>
__device__ __forceinline__ void head_mfma(const u32x4 (&buf)[GRP], const bf16_t* const (&xp)[NB], int kofs,
                                          f32x4 (&acc)[NB]) {
  u32x4 x[GRP][NB];
#pragma unroll
  for (int u = 0; u < GRP; ++u)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      x[u][nb] = *reinterpret_cast<const u32x4*>(xp[nb] + kofs + 32 * S * u);
#pragma unroll
  for (int u = 0; u < GRP; ++u)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma16x16x32(buf[u], x[u][nb], acc[nb]);
}

// Running row statistics of the lane: one (max, sum, argmax) per column block, for
// X row nb * CPB + r / S (kept by the lanes with r % S == 0).
template <int NB>
struct HeadStats {
  float m[NB], s[NB];
  int a[NB];
};

// Finish a tile: sum the S partials of every useful output entry, keep the products
// in LDS (sL[m * nloc + lt * TR + w]) and fold them into the running statistics.
// v0: vocab index of the tile's first row (statistics only).
template <int S, int NB>
__device__ __forceinline__ void head_tile_done(f32x4 (&acc)[NB], float* sL, int nloc, int M, int lt, int r, int g,
                                               bool stats, int v0, int N0, float c, HeadStats<NB>& st) {
  constexpr int TR = 16 / S, CPB = 16 / S;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int m = nb * CPB + r / S;
#pragma unroll
    for (int t = 0; t < 4 / S; ++t) {
      // lane (c = r, g) holds rows 4g + e; entry e is useful when e % S == r % S
      float v = acc[nb][0];
      const int e = r % S + S * t;
#pragma unroll
      for (int ee = 1; ee < 4; ++ee)
        if (e == ee) v = acc[nb][ee];
      if (S >= 2) v += dpp<DPP_XOR1>(v);
      if (S >= 4) v += dpp<DPP_XOR2>(v);
      const int w = (4 * g) / S + t;
      if (r % S == 0 && m < M) {
        sL[m * nloc + lt * TR + w] = v;
        if (stats && v0 + w < N0) merge_stat(st.m[nb], st.s[nb], st.a[nb], v, c != 0.0f ? 1.0f : 0.0f, v0 + w, c);
      }
    }
    acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Local index of vocab entry x in workgroup wg's products, or -1 if another owns it.
__device__ __forceinline__ int head_local_index(int x, int TR, int grid, int wg) {
  const int t = x / TR;
  const int span = grid * HEAD_WAVES;
  if ((t % span) / HEAD_WAVES != wg) return -1;
  const int lt = (t / span) * HEAD_WAVES + t % HEAD_WAVES;
  return lt * TR + x % TR;
}

__device__ __forceinline__ unsigned atomic_add_agent(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned load_coherent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_coherent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __uint_as_float(load_coherent(reinterpret_cast<const unsigned*>(p)));
}
// (m, s, a) of a partial written by another workgroup: (m, s) as one 8-byte load.
__device__ __forceinline__ void load_part_coherent(const RowPart* q, float& m, float& s, int& a) {
  const unsigned long long ms =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  m = __uint_as_float(unsigned(ms));
  s = __uint_as_float(unsigned(ms >> 32));
  a = load_coherent(&q->a);
}

__device__ __forceinline__ void put_tagged(unsigned long long* p, unsigned bits, unsigned ep) {
  __hip_atomic_store(p, (static_cast<unsigned long long>(ep) << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get_tagged(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(unsigned long long w, unsigned ep) { return unsigned(w >> 32) == ep; }

// Two-level count, thread 0 only: the workgroup's group counter (blockIdx % groups)
// and, for the last member of a group, the top counter.  Returns the top count after
// this workgroup's contribution, or 0 if it did not reach the top.  A group's last
// member resets its group counter (all members have counted).
__device__ __forceinline__ unsigned count_two_level(unsigned* cnt, int grp_word, int top_word) {
  const unsigned G = min(gridDim.x, unsigned(CNT_GROUPS));
  const unsigned g = blockIdx.x % G;
  const unsigned gsize = (gridDim.x - g + G - 1) / G;
  unsigned* gc = cnt + grp_word + g * CNT_LINE;
  if (atomic_add_agent(gc, 1u) != gsize - 1) return 0u;
  atomic_store_agent(gc, 0u);
  return atomic_add_agent(cnt + top_word, 1u) + 1u;
}

// Whether the calling workgroup is the last of the grid to pass this point (two-level
// count).  Each workgroup first waits for its own stores (the handed-over data is
// written with store_coherent, so completion means it reached the coherent side).
// The last one resets the top counter and issues an acquire fence before reading.
__device__ __forceinline__ bool last_workgroup_2l(unsigned* cnt, int grp_word, int top_word) {
  __shared__ unsigned s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned G = min(gridDim.x, unsigned(CNT_GROUPS));
    const bool last = count_two_level(cnt, grp_word, top_word) == G;
    if (last) atomic_store_agent(cnt + top_word, 0u);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// Raw bits of q[qrow + vb + e], e < 4 (bf16 zero-extended or float32), clamped to V - 1.
// (One 8- or 16-byte load where aligned measured no faster: 129.1-130.0 us per step.)
__device__ __forceinline__ void load_q4(const AcceptArgs& ac, size_t qrow, int vb, unsigned (&o)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int v = min(vb + e, ac.V - 1);
    o[e] = ac.q_bf16 ? unsigned(reinterpret_cast<const bf16_t*>(ac.q)[qrow + v])
                     : __float_as_uint(reinterpret_cast<const float*>(ac.q)[qrow + v]);
  }
}
__device__ __forceinline__ float q_value(const AcceptArgs& ac, unsigned raw) {
  return ac.q_bf16 ? __uint_as_float(raw << 16) : __uint_as_float(raw);
}

constexpr int HEAD_STAGE = 16;   // X pieces per thread in flight while staging
constexpr int HEAD_STAGE_F = 12; // the same when X is normalised from float32 rows (K = 4096: one round)
// Vocab index of the first entry of the thread's k-th group of four (or >= V).
__device__ __forceinline__ int head_group_v(int k, int nloc, int TR) {
  const int j0 = 4 * (threadIdx.x + k * blockDim.x);
  if (j0 >= nloc) return 0x7fffffff;
  const int lt = j0 / TR;
  return head_global_tile(blockIdx.x, lt, gridDim.x) * TR + (j0 - lt * TR);
}

// Gumbel noise G = -log(-log U) of the four vocab entries vb .. vb+3 at absolute
// position pos of sequence b (Philox block vb / 4, tag 1).  U lies in [2^-24, 1 - 2^-24],
// so -ln U lies in [6e-8, 16.7]: both logarithms take normal arguments and the bare
// hardware base-2 logarithm serves (no rescaling of denormal inputs).  The block index
// and the sequence are below 2^32, which saves the first round two partial products.
__device__ __forceinline__ void gumbel4(uint64_t seed, int b, uint64_t pos, int vb, float (&G)[4]) {
  const Philox4 w = philox4x64_10(uint64_t(unsigned(vb) >> 2), pos, uint64_t(unsigned(b)), TAG_GUMBEL, seed, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float nl = -LN2 * __builtin_amdgcn_logf(gumbel_uniform_from_word(w.w[e]));   // -ln U
    G[e] = -LN2 * __builtin_amdgcn_logf(nl);
  }
}

// Loads of one staging round of head_stage_norm: HEAD_STAGE_F pieces of 8 values per
// thread (the rows of Xf and the gain).  A wavefront skips a piece slot only when none of
// its lanes has a piece there (a uniform test); otherwise every lane loads, from a
// clamped in-bounds address, straight into the zeroed registers, and the conversion
// zeroes what lies outside the rows and past K.  Loads behind per-lane branches, or
// whose values are selected right away, make the compiler wait for every older load
// there (here: the stream's first weights).
__device__ __forceinline__ void head_norm_issue(const HeadArgs& a, int t0, int pieces, int kpieces, int total,
                                                f32x4 (&x0)[HEAD_STAGE_F], f32x4 (&x1)[HEAD_STAGE_F],
                                                u32x4 (&gw)[HEAD_STAGE_F]) {
  const int wbase = __builtin_amdgcn_readfirstlane(t0 - (int(threadIdx.x) & 63));   // the wavefront's lane 0
#pragma unroll
  for (int u = 0; u < HEAD_STAGE_F; ++u) {
    const int t = t0 + u * int(blockDim.x), row = t / pieces, c = t - row * pieces;
    x0[u] = x1[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    gw[u] = u32x4{0u, 0u, 0u, 0u};
    if (wbase + u * int(blockDim.x) < total) {
      const float* xr = a.Xf + size_t(min(row, a.M - 1)) * a.K + min(c, kpieces - 1) * 8;
      x0[u] = *reinterpret_cast<const f32x4*>(xr);
      x1[u] = *reinterpret_cast<const f32x4*>(xr + 4);
      gw[u] = load16(a.norm_w + min(c, kpieces - 1) * 8);
    }
  }
}

// One staging round of bf16 rows taken as they are (HEAD_STAGE pieces per thread):
// loads as in head_norm_issue, then the stores (zeros outside the rows and past K).
__device__ __forceinline__ void head_plain_issue(const HeadArgs& a, int t0, int pieces, int kpieces, int total,
                                                 u32x4 (&v)[HEAD_STAGE]) {
  const int wbase = __builtin_amdgcn_readfirstlane(t0 - (int(threadIdx.x) & 63));   // the wavefront's lane 0
#pragma unroll
  for (int u = 0; u < HEAD_STAGE; ++u) {
    const int t = t0 + u * int(blockDim.x), row = t / pieces, c = t - row * pieces;
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (wbase + u * int(blockDim.x) < total)
      v[u] = load16(a.X + size_t(min(row, a.M - 1)) * a.K + min(c, kpieces - 1) * 8);
  }
}

__device__ __forceinline__ void head_plain_store(const HeadArgs& a, int t0, int pieces, int kpieces, int total,
                                                 const u32x4 (&v)[HEAD_STAGE], bf16_t* sX, int ld) {
#pragma unroll
  for (int u = 0; u < HEAD_STAGE; ++u) {
    const int t = t0 + u * int(blockDim.x), row = t / pieces, c = t - row * pieces;
    if (t < total)
      *reinterpret_cast<u32x4*>(sX + row * ld + c * 8) = (row < a.M && c < kpieces) ? v[u] : u32x4{0u, 0u, 0u, 0u};
  }
}

// One staging round's conversion: normalise, scale by the gain, round to bf16 and store
// to LDS (zeros outside the rows and past K).
__device__ __forceinline__ void head_norm_convert(const HeadArgs& a, int t0, int pieces, int kpieces, int total,
                                                  const float* s_scale, const f32x4 (&x0)[HEAD_STAGE_F],
                                                  const f32x4 (&x1)[HEAD_STAGE_F], const u32x4 (&gw)[HEAD_STAGE_F],
                                                  bf16_t* sX, int ld) {
  const int M = a.M;
#pragma unroll
  for (int u = 0; u < HEAD_STAGE_F; ++u) {
    const int t = t0 + u * int(blockDim.x), row = t / pieces, c = t - row * pieces;
    if (t < total) {
      const bool in = row < M && c < kpieces;
      const float sc = row < M ? s_scale[row] : 0.0f;
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float xa = w < 2 ? x0[u][2 * w] : x1[u][2 * w - 4];
        const float xb = w < 2 ? x0[u][2 * w + 1] : x1[u][2 * w - 3];
        const float ga = __uint_as_float(gw[u][w] << 16), gb = __uint_as_float(gw[u][w] & 0xffff0000u);
        o[w] = in ? uint32_t(f32_to_bf16(xa * sc * ga)) | (uint32_t(f32_to_bf16(xb * sc * gb)) << 16) : 0u;
      }
      *reinterpret_cast<u32x4*>(sX + row * ld + c * 8) = o;
    }
  }
}

// X staged from float32 rows with RMSNorm: each row's scale 1 / sqrt(sum(x^2) / K + eps)
// comes from the ss_parts partial sums the producer of the rows left, summed in a fixed
// order (thread t adds parts t, t + 256, ...; then the wavefronts, then the four wave
// sums in order); every piece is normalised, scaled by the gain and rounded to bf16 as it
// is written to LDS (zeros past K and in the extra row).  The arithmetic matches a
// separate RMSNorm pass: bf16((x * scale) * g).  The first round of X loads goes out
// before the partial sums are read, so the two round trips overlap, and both go out
// before the stream's first work items (HeadFirst): vector loads complete in issue
// order, so staging loads requested after the weights would wait for them, HBM reads
// queued behind the whole chip's stream.
template <int S, int NB, int GRP, bool PAIRABLE>
__device__ __forceinline__ void head_stage_norm(const HeadArgs& a, bf16_t* sX, int ld, int Kp, const HeadFirst& hf,
                                                u32x4 (&bufA)[GRP], u32x4 (&bufB)[GRP]) {
  __shared__ float s_scale[HEAD_MAX_ROWS];
  __shared__ float s_red[HEAD_WAVES][HEAD_MAX_ROWS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = a.M;
  const int pieces = Kp / 8, kpieces = a.K / 8, total = (M + 1) * pieces;
  f32x4 x0[HEAD_STAGE_F], x1[HEAD_STAGE_F];
  u32x4 gw[HEAD_STAGE_F];
  head_norm_issue(a, threadIdx.x, pieces, kpieces, total, x0, x1, gw);
  // rows are reduced up to MR, the rows the launch's column blocks cover (M <= MR), all
  // of them unconditionally: a load whose only use sits behind the uniform test m < M is
  // moved into that branch, and each such load then waits for every older load in turn
  constexpr int MR = (16 / S) * NB < HEAD_MAX_ROWS ? (16 / S) * NB : HEAD_MAX_ROWS;
  // (rows past M and threads past ss_parts load a clamped partial, replaced by zero in
  // the reduction, where the loaded values are first used)
  float part[MR];
  {
    const int pc = min(int(threadIdx.x), a.ss_parts - 1);      // ss_parts >= 1 with a norm
#pragma unroll
    for (int m = 0; m < MR; ++m) part[m] = a.ss_in[size_t(pc) * M + min(m, M - 1)];
  }
  head_first_loads<S, NB, GRP, PAIRABLE>(a, hf, bufA, bufB);
  for (int p0 = int(blockDim.x); p0 < a.ss_parts; p0 += int(blockDim.x)) {
    const int p = p0 + int(threadIdx.x);
#pragma unroll
    for (int m = 0; m < MR; ++m)
      if (m < M && p < a.ss_parts) part[m] += a.ss_in[size_t(p) * M + m];
  }
  // rows below TR * (NB - 1) + 1 exist in every launch of this instantiation; the rest
  // only when M reaches them (their loads then wait for the weights: B * (gamma + 1)
  // just past a multiple of TR)
  constexpr int MSURE = (16 / S) * (NB - 1) + 1 < MR ? (16 / S) * (NB - 1) + 1 : MR;
  const bool own = int(threadIdx.x) < a.ss_parts;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    if (m < MSURE || m < M) {
      const float v = wave_allsum((own && m < M) ? part[m] : 0.0f);
      if (lane == 0) s_red[wave][m] = v;
    }
  }
  __syncthreads();
  if (int(threadIdx.x) < M) {
    const int m = threadIdx.x;
    const float ss = ((s_red[0][m] + s_red[1][m]) + s_red[2][m]) + s_red[3][m];
    s_scale[m] = 1.0f / sqrtf(ss / float(a.K) + a.eps);
  }
  __syncthreads();
  // the first round outside the loop: inside it, the wait for the rows would also cover
  // the later rounds' loads, which go out after the weights
  head_norm_convert(a, threadIdx.x, pieces, kpieces, total, s_scale, x0, x1, gw, sX, ld);
  for (int base = HEAD_STAGE_F * int(blockDim.x); base < total; base += HEAD_STAGE_F * int(blockDim.x)) {
    head_norm_issue(a, base + int(threadIdx.x), pieces, kpieces, total, x0, x1, gw);
    head_norm_convert(a, base + int(threadIdx.x), pieces, kpieces, total, s_scale, x0, x1, gw, sX, ld);
  }
}

// Merge of (max, sum of exp2((l - max) * c), lowest argmax) partials over groups of W
// aligned lanes (W = 8 or 64) in two passes: the group maximum, then every lane rescales
// its own sum once, and the group adds the rescaled sums and keeps the lowest index among
// the lanes holding the maximum.  Each step combines the same two operands on both
// sides, so every lane of a group ends with the same bits; the result does not depend
// on which lane holds which partial beyond the fixed butterfly order.
// Wave-wide all-reduces in two stages: DPP butterflies within each row of 16 lanes,
// then the four row values read into scalar registers and combined in a fixed order
// ((row 0, row 1), (row 2, row 3)), so every lane ends with the same bits.  Cheaper than
// lane shuffles through the LDS crossbar.  All 64 lanes must be active.
__device__ __forceinline__ float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
__device__ __forceinline__ float wave_max_rl(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  v = fmaxf(v, dpp<DPP_XOR2>(v));
  v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp<DPP_MIRROR>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_rl(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  v += dpp<DPP_MIRROR>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ int wave_min_rl(int v) {
  v = min(v, dpp<DPP_XOR1>(v));
  v = min(v, dpp<DPP_XOR2>(v));
  v = min(v, dpp<DPP_HALF_MIRROR>(v));
  v = min(v, dpp<DPP_MIRROR>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Merge of (max, sum of exp2((l - max) * c), lowest argmax) partials over groups of W
// aligned lanes (W = 8 or 64) in two passes: the group maximum, then every lane rescales
// its own sum once, and the group adds the rescaled sums and keeps the lowest index among
// the lanes holding the maximum.  Every lane of a group ends with the same bits; the
// result does not depend on the order the partials arrived in, only on their lanes.
template <int W>
__device__ __forceinline__ void group_merge_stat(float& m, float& s, int& a, float c) {
  static_assert(W == 8 || W == 64, "group of 8 lanes or the whole wave");
  float mx;
  if (W == 64) {
    mx = wave_max_rl(m);
  } else {
    mx = fmaxf(m, dpp<DPP_XOR1>(m));
    mx = fmaxf(mx, dpp<DPP_XOR2>(mx));
    mx = fmaxf(mx, dpp<DPP_HALF_MIRROR>(mx));
  }
  float t = (c != 0.0f && s != 0.0f) ? s * exp2f((m - mx) * c) : 0.0f;
  int ai = m == mx ? a : 0x7fffffff;
  if (W == 64) {
    t = wave_sum_rl(t);
    ai = wave_min_rl(ai);
  } else {
    t += dpp<DPP_XOR1>(t);
    ai = min(ai, dpp<DPP_XOR1>(ai));
    t += dpp<DPP_XOR2>(t);
    ai = min(ai, dpp<DPP_XOR2>(ai));
    t += dpp<DPP_HALF_MIRROR>(t);
    ai = min(ai, dpp<DPP_HALF_MIRROR>(ai));
  }
  m = mx;
  s = t;
  a = ai;
}

// Slice winners of the sampling launch as one orderable 64-bit key: bit 63 the class
// (1: a winner of the residual max(0, p - q), 0: a winner under p), bits 62..31 the
// score mapped to an unsigned order (-0 taken as +0), bits 30..0 the complement of the
// index, so that the largest key is the best class, then the highest score, then the
// lowest index.  Every real score maps above zero, so key 0 means "none".
__device__ __forceinline__ unsigned long long win_key(bool cls, float score, int idx) {
  const unsigned u = __float_as_uint(score + 0.0f);
  const unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(cls) << 63) | (static_cast<unsigned long long>(o) << 31) |
         static_cast<unsigned long long>(0x7fffffffu - unsigned(idx));
}
__device__ __forceinline__ int win_index(unsigned long long key) { return int(0x7fffffffu - unsigned(key & 0x7fffffffu)); }
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max_u64(unsigned long long k) {
  const unsigned lo = unsigned(dpp<CTRL>(int(unsigned(k)))), hi = unsigned(dpp<CTRL>(int(unsigned(k >> 32))));
  const unsigned long long k2 = (static_cast<unsigned long long>(hi) << 32) | lo;
  return k2 > k ? k2 : k;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long k, int l) {
  const unsigned lo = unsigned(__builtin_amdgcn_readlane(int(unsigned(k)), l));
  const unsigned hi = unsigned(__builtin_amdgcn_readlane(int(unsigned(k >> 32)), l));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }
__device__ __forceinline__ unsigned long long wave_allmax_u64(unsigned long long k) {
  k = dpp_max_u64<DPP_XOR1>(k);
  k = dpp_max_u64<DPP_XOR2>(k);
  k = dpp_max_u64<DPP_HALF_MIRROR>(k);
  k = dpp_max_u64<DPP_MIRROR>(k);
  return max_u64(max_u64(readlane_u64(k, 0), readlane_u64(k, 16)), max_u64(readlane_u64(k, 32), readlane_u64(k, 48)));
}

// PAIRABLE: the instantiation that honours write_out == 2 (the decoder's products use it for
// all their launches, paired or not, so that they share one kernel's code).
template <int S, int NB, int GRP, bool PAIRABLE = false>
__global__ __launch_bounds__(HEAD_WAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_head(HeadArgs a) {
  constexpr int TR = 16 / S, CPB = 16 / S;
  constexpr int NW = HEAD_WAVES;
  // K need not be a multiple of the work item: the last item of a tile runs past the
  // row into the next row's bytes (or past the segment's end, read as zeros), and X
  // holds zeros there, so those products add nothing.
  const int Kp = a.gpt * GRP * 32 * S;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sX = reinterpret_cast<bf16_t*>(smem);
  float* sL = reinterpret_cast<float*>(smem + head_lds_x(a.M, Kp, S));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int ld = Kp + 8 * S;
  const int ntiles = a.tile_end[a.nseg - 1];
  const int M = a.M, nloc = a.nloc, N0 = a.N[0];
  const AcceptArgs& ac = a.acc;
  const bool rule = a.mode != HEAD_PRODUCT;
  const bool sample = a.mode == HEAD_SAMPLE;
  const bool stats = a.part != nullptr;
  const int G1 = ac.gamma + 1;

  // per-row inputs of the rule, fetched before the stream (their latency would
  // otherwise land after it, behind the other workgroups' traffic)
  __shared__ int s_draft[HEAD_MAX_ROWS];
  __shared__ float s_qx[HEAD_MAX_ROWS], s_u[HEAD_MAX_ROWS];
  __shared__ int s_bad[HEAD_MAX_ROWS];
  __shared__ long long s_pos0[HEAD_MAX_ROWS];
  __shared__ unsigned s_ep;                       // HEAD_SAMPLE: this launch's epoch

  // What the staging waits for is requested before the wavefront's first two work items:
  // the first round of X (and the norm's partial sums), then the two items, then the
  // rule's per-row inputs and the launch epoch.  Vector loads complete in issue order, so
  // loads requested after the weights would wait for them; this way the stream starts two
  // items deep while X is converted and stored.
  const int first = blockIdx.x * HEAD_WAVES + wave, tstride = gridDim.x * HEAD_WAVES;
  const bool pair = PAIRABLE && a.write_out == 2;
  const int n_my = head_tiles_of(a, first, tstride, ntiles, pair);
  const int psh = pair ? 1 : 0;
  const int slot = psh ? head_pair_slot(first, gridDim.x) : first;
  const int items = n_my * a.gpt;
  const int item_k = 32 * S * GRP;                // elements of a row per work item
  const int lane_ofs = 8 * (S * g + r % S);       // element offset of the lane's piece in step 0
  int my_draft = -1, my_bad = 0;
  long long my_pos0 = 0, my_pos0_row = 0;        // pos0 of sequence threadIdx.x, of row threadIdx.x's sequence
  unsigned my_ep = 0u;
  // The rule's inputs, requested after the first round of X and the stream's first two
  // work items: loads complete in issue order, so the staging waits only for X (the
  // epoch is a load that bypasses the caches; requested before X, the staging waited for
  // it) and the stream's later waits find them arrived.
  auto rule_inputs = [&]() {
    if (rule && threadIdx.x < M) {
      const int b = threadIdx.x / G1, i = threadIdx.x - b * G1;
      if (i < ac.gamma) my_draft = ac.draft[size_t(b) * ac.draft_stride + ac.draft_offset + i];
      if (sample) my_pos0_row = ac.pos0[b];
    }
    if (sample && threadIdx.x < ac.B) {
      my_pos0 = ac.pos0[threadIdx.x];
      my_bad = ac.invalid ? ac.invalid[threadIdx.x] : 0;
    }
    if (sample && threadIdx.x == 0) my_ep = load_coherent(a.counter + CNT_EPOCH);
  };
  const HeadFirst hf{items, slot, psh, tstride, item_k, ntiles,
                     (unsigned(r / S) * unsigned(a.K) + unsigned(lane_ofs)) * 2u};   // the lane's W bytes
  const unsigned voff = hf.voff;
  u32x4 bufA[GRP], bufB[GRP];

  // stage all of X (zeros from K to Kp) and the zero row, HEAD_STAGE pieces per thread
  // in flight at a time (one load and store at a time would chain the L2 round trips)
  if (a.Xf) {
    rule_inputs();
    head_stage_norm<S, NB, GRP, PAIRABLE>(a, sX, ld, Kp, hf, bufA, bufB);
  } else {
    const int pieces = Kp / 8, kpieces = a.K / 8, total = (M + 1) * pieces;
    // the first round's loads, then the stream's first work items and the rule's inputs,
    // then its stores; the later rounds (long or many rows) after
    u32x4 v[HEAD_STAGE];
    head_plain_issue(a, threadIdx.x, pieces, kpieces, total, v);
    head_first_loads<S, NB, GRP, PAIRABLE>(a, hf, bufA, bufB);
    rule_inputs();
    head_plain_store(a, threadIdx.x, pieces, kpieces, total, v, sX, ld);
    for (int base = HEAD_STAGE * int(blockDim.x); base < total; base += HEAD_STAGE * int(blockDim.x)) {
      head_plain_issue(a, base + int(threadIdx.x), pieces, kpieces, total, v);
      head_plain_store(a, base + int(threadIdx.x), pieces, kpieces, total, v, sX, ld);
    }
  }
  __syncthreads();

  const bf16_t* xp[NB];                           // the lane's X row in each column block
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) xp[nb] = sX + min(nb * CPB + r / S, M) * ld + lane_ofs;

  // sampling: q at each draft token and the acceptance uniforms, while the first loads fly
  float my_qx = 0.0f;
  if (sample && threadIdx.x < M) {
    const int t = threadIdx.x, b = t / G1, i = t - b * G1;
    const int x = my_draft;
    if (x >= 0 && x < ac.V) {
      const size_t qi = (size_t(b) * ac.gamma + i) * ac.V + x;
      my_qx = ac.q_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(ac.q)[qi])
                        : reinterpret_cast<const float*>(ac.q)[qi];
    }
    s_u[t] = i < ac.gamma ? accept_uniform(ac.seed, uint64_t(b), uint64_t(my_pos0_row + i + 1)) : 1.0f;
  }

  const int kg = (nloc / 4 + int(blockDim.x) - 1) / int(blockDim.x);   // groups of four per thread
  // q of the residual draw is read in the draw, for row n only.  Prefetched here for every
  // drafted row (2 MB a step, issued ahead of the stream), it delayed the stream's first
  // loads: 131.8-132.0 against 128.7-129.9 us per step.

  HeadStats<NB> st;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) { st.m[nb] = -INFINITY; st.s[nb] = 0.0f; st.a[nb] = 0x7fffffff; }
  const float c = a.c_stat;
  if (items > 0) {
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    int k = 0;
#define SV_HEAD_ITEM(KK, BUF)                                                                             \
    {                                                                                                     \
      const int i_ = (KK) / a.gpt, gg_ = (KK) - i_ * a.gpt;                                               \
      head_mfma<S, NB, GRP>(BUF, xp, gg_ * item_k, acc);                                                  \
      if (gg_ == a.gpt - 1) {                                                                             \
        head_tile_done<S, NB>(acc, sL, nloc, M, i_ * HEAD_WAVES + wave, r, g, stats,                      \
                              (first + i_ * tstride) * TR, N0, c, st);                                    \
      }                                                                                                   \
    }
    // items k (bufA) and k + 1 (bufB) are in flight at the top of each iteration
    for (; k + 3 < items; k += 2) {
      SV_HEAD_ITEM(k, bufA)
      head_load<S, NB, GRP>(head_item<S, PAIRABLE>(a, k + 2, slot, psh, tstride, item_k), voff, bufA);
      SV_HEAD_ITEM(k + 1, bufB)
      head_load<S, NB, GRP>(head_item<S, PAIRABLE>(a, k + 3, slot, psh, tstride, item_k), voff, bufB);
    }
    if (k + 2 < items) {
      SV_HEAD_ITEM(k, bufA)
      head_load<S, NB, GRP>(head_item<S, PAIRABLE>(a, k + 2, slot, psh, tstride, item_k), voff, bufA);
      SV_HEAD_ITEM(k + 1, bufB)
      SV_HEAD_ITEM(k + 2, bufA)
    } else if (k + 1 < items) {
      SV_HEAD_ITEM(k, bufA)
      SV_HEAD_ITEM(k + 1, bufB)
    } else {
      SV_HEAD_ITEM(k, bufA)
    }
#undef SV_HEAD_ITEM
  }
  if (sample && threadIdx.x < M) s_qx[threadIdx.x] = my_qx;
  // the rule's per-row inputs, requested before the stream; the barrier below publishes them
  if (rule && threadIdx.x < M) s_draft[threadIdx.x] = my_draft;
  if (sample && threadIdx.x < ac.B) {
    s_pos0[threadIdx.x] = my_pos0;
    s_bad[threadIdx.x] = my_bad;
  }
  if (sample && threadIdx.x == 0)
    s_ep = my_ep == EPOCH_POISON ? my_ep : (my_ep + 1u >= EPOCH_POISON ? 1u : my_ep + 1u);   // 0 never tags a record

  // ---- statistics partials: lanes of a row differ in g (xor 16, 32), then the waves
  __shared__ float s_m[HEAD_WAVES][HEAD_MAX_ROWS], s_s[HEAD_WAVES][HEAD_MAX_ROWS];
  __shared__ int s_a[HEAD_WAVES][HEAD_MAX_ROWS];
  if (stats) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      xor_merge_stat(st.m[nb], st.s[nb], st.a[nb], c, 16);
      xor_merge_stat(st.m[nb], st.s[nb], st.a[nb], c, 32);
      const int m = nb * CPB + r / S;
      if (g == 0 && r % S == 0 && m < M) { s_m[wave][m] = st.m[nb]; s_s[wave][m] = st.s[nb]; s_a[wave][m] = st.a[nb]; }
    }
  }
  __syncthreads();

  const int tpw = nloc / TR;                      // local tiles per workgroup
  // ---- write the products (residual: add them into out, and leave each tile's sum of
  // squares of the updated entries in its first LDS slot, summed per row below in
  // tile order)
  if (pair) {
    // gate tile of round 2u (local tile lt) and up tile of round 2u + 1 (lt + HEAD_WAVES):
    // the same rows, the same formula as the separate SwiGLU kernel
    for (int idx = threadIdx.x; idx < M * tpw; idx += blockDim.x) {
      const int m = idx / tpw, lt = idx - m * tpw;
      const int i = lt / HEAD_WAVES, f = blockIdx.x * HEAD_WAVES + lt % HEAD_WAVES;
      if ((i & 1) || 2 * (i >> 1) >= head_tiles_of(a, f, gridDim.x * HEAD_WAVES, ntiles, true)) continue;
      const TileRef tr = head_tile_pair(a, head_global_tile(blockIdx.x, lt, gridDim.x), TR);
      const float* gs = sL + m * nloc + lt * TR;
      const float* us = gs + HEAD_WAVES * TR;
      bf16_t* dst = a.hout + size_t(m) * tr.N + tr.v0;
      for (int w = 0; w < TR && tr.v0 + w < tr.N; ++w) {
        const float gv = gs[w];
        dst[w] = f32_to_bf16(gv / (1.0f + expf(-gv)) * us[w]);
      }
    }
  } else if (a.write_out) {
    const bool res = a.residual != 0;
    for (int idx = threadIdx.x; idx < M * tpw; idx += blockDim.x) {
      const int m = idx / tpw, lt = idx - m * tpw;
      const int t = head_global_tile(blockIdx.x, lt, gridDim.x);
      float* src = sL + m * nloc + lt * TR;
      if (t >= ntiles) {
        if (res) src[0] = 0.0f;
        continue;
      }
      const TileRef tr = head_tile(a, t, TR);
      float* dst = tr.out + size_t(m) * tr.N + tr.v0;
      float ssq = 0.0f;
      if (tr.v0 + TR <= tr.N && (tr.N & 3) == 0 && (reinterpret_cast<uintptr_t>(tr.out) & 15) == 0) {
#pragma unroll
        for (int q = 0; q < TR; q += 4) {
          f32x4 v = *reinterpret_cast<const f32x4*>(src + q);
          if (res) {
            v += *reinterpret_cast<const f32x4*>(dst + q);
#pragma unroll
            for (int e = 0; e < 4; ++e) ssq = fmaf(v[e], v[e], ssq);
          }
          *reinterpret_cast<f32x4*>(dst + q) = v;
        }
      } else {
        for (int w = 0; w < TR && tr.v0 + w < tr.N; ++w) {
          float v = src[w];
          if (res) { v += dst[w]; ssq = fmaf(v, v, ssq); }
          dst[w] = v;
        }
      }
      if (res) src[0] = ssq;
    }
    if (res && a.ss_out) {
      __syncthreads();
      for (int m = threadIdx.x; m < M; m += blockDim.x) {
        float ss = 0.0f;
        for (int lt = 0; lt < tpw; ++lt) ss += sL[m * nloc + lt * TR];
        a.ss_out[size_t(blockIdx.x) * M + m] = ss;
      }
    }
  }
  if (!stats) return;

  if (!sample) {
    for (int m = threadIdx.x; m < M; m += blockDim.x) {
      float rm = -INFINITY, rs = 0.0f;
      int ra = 0x7fffffff;
#pragma unroll
      for (int w = 0; w < HEAD_WAVES; ++w) merge_stat(rm, rs, ra, s_m[w][m], s_s[w][m], s_a[w][m], c);
      store_part(a.part + size_t(blockIdx.x) * M + m, rm, rs, ra);
      // draft-token logit of this row, if this workgroup holds it
      if (rule && a.xlogit) {
        const int x = s_draft[m];
        if (x >= 0 && x < N0) {
          const int j = head_local_index(x, TR, gridDim.x, blockIdx.x);
          if (j >= 0) store_coherent(a.xlogit + m, sL[m * nloc + j]);
        }
      }
    }
    if (!rule) return;
    if (last_workgroup_2l(a.counter, CNT_GRP_ARRIVE, CNT_TOP_ARRIVE)) accept_block(ac, 0, ac.B);
    return;
  }

  // ---- HEAD_SAMPLE.  Every hand-off is a set of epoch-tagged words that the reader
  // polls (bounded) until all carry this launch's epoch:
  //   1. each workgroup publishes its statistics partial (and the draft logits it holds);
  //   2. the first workgroup of each XCD group merges its group's partials and
  //      publishes a group partial;
  //   3. every workgroup reads the G group partials, decides n for every sequence
  //      (same inputs, same arithmetic, same n), draws the Gumbel-max of row n over its
  //      slice and publishes its slice winner;
  //   4. workgroup 0 merges the winners, writes the outputs and stores the epoch.
  // A wait that times out makes the step report every sequence invalid.  Workgroup 0
  // still advances the stored epoch if every workgroup has published its statistics
  // record (so every one of them read the epoch), and the next launch -- which starts
  // after every workgroup of this one has ended -- ignores the records this one left.
  // Only if some workgroup had not published (the device could not hold the whole grid)
  // does it mark the workspace, so that such a late workgroup publishes nothing; calls
  // on that workspace then report every sequence invalid until it is zero-filled.
  const unsigned ep = s_ep;
  const unsigned G = min(gridDim.x, unsigned(CNT_GROUPS));
  const int RG = a.rec_grid;
  unsigned long long* r_part = a.recs;                                  // [RG][M][4]
  unsigned long long* r_group = r_part + size_t(RG) * M * 4;            // [8][M][4]
  unsigned long long* r_xl = r_group + size_t(CNT_GROUPS) * M * 4;      // [M]
  unsigned long long* r_win = r_xl + M;                                 // [B][RG][4]
  if (ep == EPOCH_POISON) {
    if (blockIdx.x == 0)
      for (int b = threadIdx.x; b < ac.B; b += blockDim.x) {
        for (int i = 0; i < G1; ++i) ac.tokens_out[b * G1 + i] = -1;
        ac.n_accepted[b] = -1;
      }
    return;
  }
  __shared__ int s_ok;
  if (threadIdx.x == 0) s_ok = 1;
  __syncthreads();

  // 1. publish the partial and the draft logits this workgroup holds
  for (int m = threadIdx.x; m < M; m += blockDim.x) {
    float rm = -INFINITY, rs = 0.0f;
    int ra = 0x7fffffff;
#pragma unroll
    for (int w = 0; w < HEAD_WAVES; ++w) merge_stat(rm, rs, ra, s_m[w][m], s_s[w][m], s_a[w][m], c);
    unsigned long long* rec = r_part + (size_t(blockIdx.x) * M + m) * 4;
    put_tagged(rec + 0, __float_as_uint(rm), ep);
    put_tagged(rec + 1, __float_as_uint(rs), ep);
    put_tagged(rec + 2, unsigned(ra), ep);
    const int x = s_draft[m];
    if (x >= 0 && x < N0) {
      const int j = head_local_index(x, TR, gridDim.x, blockIdx.x);
      if (j >= 0) put_tagged(r_xl + m, __float_as_uint(sL[m * nloc + j]), ep);
    }
  }

  // 2. the first workgroup of each group merges its members' partials: wave w takes
  //    rows w, w + NW, ... (all polled together), lane k member k
  if (blockIdx.x < G) {
    constexpr int RPW = (HEAD_MAX_ROWS + NW - 1) / NW;   // rows per wave
    const unsigned g = blockIdx.x, gsize = (gridDim.x - g + G - 1) / G;
    float rm[RPW], rs[RPW];
    int ra[RPW];
    unsigned spins = 0;
    bool got = false;
    for (;;) {
      bool mine = true;
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        const int m = wave + NW * j;
        rm[j] = -INFINITY; rs[j] = 0.0f; ra[j] = 0x7fffffff;
        if (m < M && unsigned(lane) < gsize) {
          const unsigned long long* rec = r_part + (size_t(g + G * lane) * M + m) * 4;
          const unsigned long long w0 = get_tagged(rec), w1 = get_tagged(rec + 1), w2 = get_tagged(rec + 2);
          mine = mine && tag_is(w0, ep) && tag_is(w1, ep) && tag_is(w2, ep);
          rm[j] = __uint_as_float(unsigned(w0)); rs[j] = __uint_as_float(unsigned(w1)); ra[j] = int(unsigned(w2));
        }
      }
      if (__all(mine)) { got = true; break; }
      if (spins++ >= a.spin_limit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (!got) {
      if (lane == 0) s_ok = 0;
    } else {
#pragma unroll
      for (int j = 0; j < RPW; ++j) group_merge_stat<64>(rm[j], rs[j], ra[j], c);
#pragma unroll
      for (int j = 0; j < RPW; ++j) {
        const int m = wave + NW * j;
        if (lane == 0 && m < M) {
          unsigned long long* out = r_group + (size_t(g) * M + m) * 4;
          put_tagged(out + 0, __float_as_uint(rm[j]), ep);
          put_tagged(out + 1, __float_as_uint(rs[j]), ep);
          put_tagged(out + 2, unsigned(ra[j]), ep);
        }
      }
    }
  }

  // 3b. read the G group partials (eight lanes per row, merged in a fixed order) and
  //     the draft logits; each wave polls its own rows
  __shared__ float s_xl[HEAD_MAX_ROWS];
  for (int row0 = wave * 8; row0 < M; row0 += 8 * NW) {
    const int row = row0 + lane / 8, gp = lane % 8;
    const bool need = row < M && unsigned(gp) < G;
    const unsigned long long* rec = r_group + (size_t(gp) * M + row) * 4;
    // the row's first lane also watches the row's draft logit
    const int x = row < M ? s_draft[row] : -1;
    const bool need_xl = gp == 0 && x >= 0 && x < N0;
    float m = -INFINITY, sm = 0.0f, xl = 0.0f;
    int am = 0x7fffffff;
    unsigned spins = 0;
    bool got = false;
    for (;;) {
      bool mine = true;
      if (need) {
        const unsigned long long w0 = get_tagged(rec), w1 = get_tagged(rec + 1), w2 = get_tagged(rec + 2);
        mine = tag_is(w0, ep) && tag_is(w1, ep) && tag_is(w2, ep);
        m = __uint_as_float(unsigned(w0)); sm = __uint_as_float(unsigned(w1)); am = int(unsigned(w2));
      }
      if (need_xl) {
        const unsigned long long w = get_tagged(r_xl + row);
        mine = mine && tag_is(w, ep);
        xl = __uint_as_float(unsigned(w));
      }
      if (__all(mine)) { got = true; break; }
      if (spins++ >= a.spin_limit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (!got) { if (lane == 0) s_ok = 0; break; }
    if (!need) { m = -INFINITY; sm = 0.0f; am = 0x7fffffff; }
    group_merge_stat<8>(m, sm, am, c);
    if (gp == 0 && row < M) { s_m[0][row] = m; s_s[0][row] = sm; s_a[0][row] = am; s_xl[row] = xl; }
  }
  __syncthreads();
  const bool ok = s_ok != 0;

  // 3c. decide n for every sequence
  __shared__ int s_n[HEAD_MAX_ROWS];
  __shared__ float s_mn[HEAD_MAX_ROWS], s_zn[HEAD_MAX_ROWS];
  if (ok) {
    for (int b = wave; b < ac.B; b += NW) {
      const int row = b * G1 + lane;
      float my_m = -INFINITY, my_s = 0.0f;
      float px = 0.0f, qx = 0.0f, u = 1.0f;
      if (lane < G1) { my_m = s_m[0][row]; my_s = s_s[0][row]; }
      if (lane < ac.gamma) {
        const int x = s_draft[row];
        u = s_u[row];
        if (x >= 0 && x < ac.V) {
          px = exp2f((s_xl[row] - my_m) * c) / my_s;
          qx = s_qx[row];
        }
      }
      const bool acc_ok = double(u) * double(qx) < double(px);   // exact: 24-bit u times <= 24-bit q
      const unsigned long long rej = __ballot(lane < ac.gamma && !acc_ok);
      const int n = rej ? __ffsll(rej) - 1 : ac.gamma;
      const float m_n = __shfl(my_m, n), z_n = __shfl(my_s, n);
      if (lane == 0) { s_n[b] = s_bad[b] ? -1 : n; s_mn[b] = m_n; s_zn[b] = z_n; }
    }
    __syncthreads();
  }

  // 3d. Gumbel-max of row n_b over this slice; publish one winner per (sequence, workgroup)
  __shared__ unsigned long long s_key[NW];
  for (int b = 0; b < ac.B && ok; ++b) {
    const int n = __builtin_amdgcn_readfirstlane(s_n[b]);   // the same for every thread
    float sr = -INFINITY, sp = -INFINITY;
    int ir = 0x7fffffff, ip = 0x7fffffff;
    if (n >= 0) {
      // log p = (l - max) * c * ln 2 - ln z exactly; p itself only for the residual
      const float mx = s_mn[b], z = s_zn[b], lnz = logf(z), inv_z = 1.0f / z;
      const bool resid = n < ac.gamma;
      const float* l = sL + (b * G1 + n) * nloc;
      const uint64_t pos = uint64_t(s_pos0[b] + n + 1);
      for (int k = 0; k < kg; ++k) {
        const int j0 = 4 * (threadIdx.x + k * blockDim.x);
        if (j0 >= nloc) break;
        const int vb = head_group_v(k, nloc, TR);
        if (vb >= ac.V) continue;
        unsigned qr[4] = {0u, 0u, 0u, 0u};
        if (resid) load_q4(ac, (size_t(b) * ac.gamma + n) * ac.V, vb, qr);
        float gn[4];
        gumbel4(ac.seed, b, pos, vb, gn);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = vb + e;
          if (v >= ac.V) break;
          const float Gv = gn[e];
          const float t = (l[j0 + e] - mx) * ac.c;
          const float scp = t * LN2 - lnz + Gv;
          if (scp > sp) { sp = scp; ip = v; }
          if (resid) {
            // where q is zero the residual is p itself: score it with p's expression, so
            // a padded slot (q = 0 everywhere) draws exactly the bonus draw's token
            const float qv = q_value(ac, qr[e]);
            const float rr = fmaxf(exp2f(t) * inv_z - qv, 0.0f);
            if (rr > 0.0f) {
              const float sc = qv == 0.0f ? scp : __logf(rr) + Gv;
              if (sc > sr) { sr = sc; ir = v; }
            }
          }
        }
      }
    }
    // the slice's residual winner if it has one (class 1), else its winner under p
    unsigned long long key = ir != 0x7fffffff ? win_key(true, sr, ir) : ip != 0x7fffffff ? win_key(false, sp, ip) : 0ull;
    key = wave_allmax_u64(key);
    if (lane == 0) s_key[wave] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < NW; ++w) key = s_key[w] > key ? s_key[w] : key;
      unsigned long long* rec = r_win + (size_t(b) * RG + blockIdx.x) * 2;
      put_tagged(rec + 0, unsigned(key >> 32), ep);
      put_tagged(rec + 1, unsigned(key), ep);
    }
    __syncthreads();
  }
  if (!ok && threadIdx.x == 0) atomic_store_agent(a.counter + CNT_FAIL, ep);

  // 4. workgroup 0 merges the winners, writes the outputs and stores the epoch
  if (blockIdx.x != 0) return;
  __shared__ int s_tok[HEAD_MAX_ROWS];
  bool done = ok;
  for (int b = 0; b < ac.B && done; ++b) {
    if (s_n[b] < 0) continue;
    // the largest slice-winner key: the residual's winner when any slice has one, else
    // the winner under p
    unsigned long long key = 0ull;
    unsigned spins = 0;
    for (;;) {
      bool mine = true;
      unsigned long long tk = 0ull;
      for (int p = threadIdx.x; p < int(gridDim.x); p += blockDim.x) {
        const unsigned long long* rec = r_win + (size_t(b) * RG + p) * 2;
        const unsigned long long w0 = get_tagged(rec), w1 = get_tagged(rec + 1);
        if (tag_is(w0, ep) && tag_is(w1, ep)) {
          const unsigned long long k2 = (static_cast<unsigned long long>(unsigned(w0)) << 32) | unsigned(w1);
          tk = k2 > tk ? k2 : tk;
        } else {
          mine = false;
        }
      }
      if (__syncthreads_and(mine)) { key = tk; break; }
      // a workgroup that gave up never publishes: stop waiting (one uniform answer)
      const bool failed = __syncthreads_or(threadIdx.x == 0 && load_coherent(a.counter + CNT_FAIL) == ep);
      if (failed || spins++ >= a.spin_limit) { done = false; break; }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!done) break;
    key = wave_allmax_u64(key);
    if (lane == 0) s_key[wave] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 1; w < NW; ++w) key = s_key[w] > key ? s_key[w] : key;
      s_tok[b] = win_index(key);
    }
    __syncthreads();
  }
  for (int b = threadIdx.x; b < ac.B; b += blockDim.x) {
    const int n = done ? s_n[b] : -1;
    for (int i = 0; i < G1; ++i) {
      int t = -1;
      if (n >= 0 && i < n) t = s_draft[b * G1 + i];
      else if (n >= 0 && i == n) t = s_tok[b];
      ac.tokens_out[b * G1 + i] = t;
    }
    ac.n_accepted[b] = n;
    if (ac.len && n >= 0) ac.len[b] += n + 1;
  }
  // every winner arrived: every workgroup has run; otherwise look for each one's
  // statistics record (published right after its stream)
  bool all_ran = done;
  if (!done) {
    bool mine = true;
    for (int p = threadIdx.x; p < int(gridDim.x); p += blockDim.x)
      mine = mine && tag_is(get_tagged(r_part + size_t(p) * M * 4), ep);
    all_ran = __syncthreads_and(mine);
  }
  if (threadIdx.x == 0) atomic_store_agent(a.counter + CNT_EPOCH, all_ran ? ep : EPOCH_POISON);
}

}  // namespace sv
