// Batch-invariant paged attention for gfx950: split phase and merge phase.
//
// What is computed (Vosti deep-dive blog (深入解析 Vosti), §6.2, attention causal
// contract): the query row at position p = k_len - q_len + i sees keys [lo, p],
// lo = max(0, p - w + 1) under a sliding window, and its output depends only on
// that row of Q and those keys and values — not on the query length, the row
// index, the batch or the physical page table.
//
// How the arithmetic of a row is fixed by logical key positions alone:
//  * keys are cut into splits of a fixed SIZE S, [sS, (s+1)S), never a fixed
//    count (record "Deterministic and bit-exact inference", field technical,
//    Invariance);
//  * a split is a pass over 32-key tiles in increasing order with an online
//    softmax (deep-dive blog, §6.2: the tiles meeting a row's range are visited
//    in the same order by every invocation);
//  * a tile where a row sees no key leaves that row's (m, l, acc) bit-for-bit
//    unchanged, by select (deep-dive blog, §6.2, value rules: masked score
//    -inf, masked weight 0, an all-false row copies its incoming state);
//  * masking is a select, never an additive bias, so keys outside [lo, p] —
//    including never-written slots holding NaN — cannot reach the result;
//    values of keys at or past k_len are zero-filled on load;
//  * decode rows and prefill rows go through the same MFMA instructions: a
//    query-row block is 16 MFMA columns = (16 / G) tokens x G heads of one KV
//    head, and a decode block simply leaves columns empty;
//  * splits are merged in increasing split order (merge kernel), and a -0
//    result is stored as +0.
//
// Data path per wave (no LDS): the K tile is read straight into the A operand
// of v_mfma_f32_16x16x32_bf16 (S^T = K Q^T), the score fragments that come out
// are exactly the B operand of the PV product (O^T = V^T P^T), and the V
// fragments are read straight into its A operand.  The cache layouts
// (K [page][h][D/8][16][8], V [page][h][D/32][16][16][2]) make every one of
// these reads a fully used contiguous KiB per wave instruction.

#include "bi_internal.h"

#include <math.h>

#include <algorithm>

namespace bi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Read of a table the split kernel never writes (page table, sequence
// metadata, work plan) through the constant address space: the compiler then
// keeps uniform reads on the scalar unit, whose waits do not touch the vector
// memory counter that tracks the K/V tiles in flight.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int ldc(const int32_t* p, int64_t i) { return ((const_i32_ptr)p)[i]; }

// Maximum over the four lanes l, l^16, l^32, l^48 that hold one query row,
// with the gfx950 lane-swap instructions (VALU only; no LDS traffic and no
// wait on the memory counters).  Swapping a value with itself and combining
// the two results gives every lane of a row the same operands in the same
// order: max(max(r0, r1), max(r2, r3)), where ri is the value of lane group i.
__device__ __forceinline__ float row4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---------------------------------------------------------------------------
// Building blocks of the split phase.
// ---------------------------------------------------------------------------

// Online-softmax state of the query row held by this lane (the four lanes of a
// row hold identical m and l).  The row sum l is the accumulator of one more
// PV-shaped product whose A operand is all ones, so all four of its entries
// hold the same l.
template <int D>
struct SplitState {
  float m;
  f32x4 lacc;
  f32x4 acc[D / 16];
  __device__ __forceinline__ float l() const { return lacc[0]; }
  __device__ __forceinline__ void init() {
    m = -INFINITY;
    lacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// A split's accumulator goes to the merge (workspace or LDS) as bf16, rounded
// to nearest even: four consecutive head-dim values per lane, 8 bytes.
__device__ __forceinline__ u32x2 acc_to_bf16(const f32x4& v) {
  bf16x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (__bf16)v[i];
  return __builtin_bit_cast(u32x2, b);
}

__device__ __forceinline__ f32x4 bf16_to_acc(const u32x2& w) {
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

// Operands of one 32-key tile (two pages of 16 keys) for this lane.
template <int D>
struct TileData {
  u32x4 kf[2][D / 32];   // K rows: A operand of S^T = K Q^T
  u32x4 vf[2][D / 32];   // V^T fragments of two head-dim blocks, interleaved (see load_tile)
  u32x2 vmask[2];        // per page: keeps the bits of this lane's keys below k_len
};

// Keys [lo, hi] of this split visible to this lane's row (empty if lo > hi).
struct RowMask {
  int lo, hi;
};

// Per-lane part of an item's query-row block: this lane's row, its visible
// keys inside the split, and its Q fragment (B operand of S^T = K Q^T: step
// st, lane group g4 holds head-dim chunk 4*st + g4).
template <int D>
struct ItemLane {
  RowMask rm;
  bf16x8 q[D / 32];
};

// Page-table entries of the two 16-key halves of a tile.  The read is
// unconditional (its index is clamped to the last entry the sequence uses, so
// entries past ceil(k_len / 16) are never read) and its result is first needed
// by the next stage, so the scalar load latency hides behind a tile compute.
__device__ __forceinline__ int2 tile_pages(const int32_t* pt_row, int last_entry, int tile) {
  return make_int2(ldc(pt_row, min(2 * tile, last_entry)), ldc(pt_row, min(2 * tile + 1, last_entry)));
}

// Cache policy of the K/V tile loads: non-temporal (each byte is read once).
constexpr int kStreamLoad = 2;

// Raw buffer resource over one page of one KV head (gfx9 word 3: 32-bit data
// format, no swizzle).  With num_records = 0 every load through it returns
// zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, bytes, 0x00020000);
}

// Issue the loads of one tile.  Every call issues the same loads (pages past
// k_len, past the page-table row or past the split go through an empty buffer
// resource and read as zero), so the number of loads in flight is static and
// the wait before a tile is computed covers only that tile's loads.  Nothing
// here reads the loaded registers.  K rows of keys at or past k_len need no
// clearing: a key's row of S^T only feeds that key's scores, which the mask
// replaces by -inf.  V of such keys must be zero (0 * NaN would reach every
// row through the PV contraction; never-written slots may hold NaN), so a
// per-page bit mask is recorded and applied when the tile is computed.
template <int D>
__device__ __forceinline__ void load_tile(const AttnSplitArgs& a, int kvh, int k_len, int tile, int tile_end,
                                          int2 pid, int lane, TileData<D>& t) {
  constexpr int NSTEP = D / 32;
  constexpr int NBLK = D / 16;
  constexpr int PAGE_BYTES = D * 16 * 2;
  (void)NSTEP;
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t head_elems = (int64_t)D * 16;
  const bool live_tile = tile < tile_end;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    // A half is read only if it lies in the split, below k_len, inside the
    // page-table row, and names a page of the pool.
    const int entry = 2 * tile + b;
    const int raw = b == 0 ? pid.x : pid.y;
    const int pgc = min(max(raw, 0), a.num_pages - 1);  // always a page of the pool
    const bool ok = live_tile && entry * 16 < k_len && entry < a.pt_stride && raw == pgc;
    const int pg = ok ? pgc : -1;
    const int nl = min(16, k_len - (tile * 32 + 16 * b)) - 4 * g4;  // valid keys among this lane's four
    t.vmask[b].x = (pg < 0) ? 0u : (nl >= 2 ? 0xffffffffu : (nl == 1 ? 0x0000ffffu : 0u));
    t.vmask[b].y = (pg < 0) ? 0u : (nl >= 4 ? 0xffffffffu : (nl == 3 ? 0x0000ffffu : 0u));
    const int64_t base = ((int64_t)pgc * a.num_kv_heads + kvh) * head_elems;
    const __amdgpu_buffer_rsrc_t kr = page_rsrc(a.k_cache + base, pg < 0 ? 0 : PAGE_BYTES);
    const __amdgpu_buffer_rsrc_t vr = page_rsrc(a.v_cache + base, pg < 0 ? 0 : PAGE_BYTES);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
      t.kf[b][st] = __builtin_amdgcn_raw_buffer_load_b128(kr, (64 * st + lane) * 16, 0, kStreamLoad);
    // V page layout [D/32][16][16][2]: head-dim d = 32*np + 16*e + r, token o at
    // ((np*16 + r)*16 + o)*2 + e.  One 16-byte load gives this lane tokens
    // 4*g4 .. 4*g4+3 of rows d = 32*np + r (e = 0) and 32*np + 16 + r (e = 1);
    // per np the 64 lanes read one contiguous KiB.
#pragma unroll
    for (int np = 0; np < NBLK / 2; ++np)
      t.vf[b][np] = __builtin_amdgcn_raw_buffer_load_b128(vr, ((np * 16 + r) * 16 + 4 * g4) * 4, 0, kStreamLoad);
  }
}

// One online-softmax step over a 32-key tile for the rows of QB query-row
// blocks (this lane's row of each).  Each phase runs over the blocks before the
// next phase starts, so the blocks' independent MFMA chains and reductions can
// overlap; every row still goes through exactly the operations, in exactly the
// order, it would alone.  A row with no visible key in the tile keeps
// (m, l, acc) bit-for-bit (select, not update).
//
// Per row, with raw scores s_k = q . k_k of the tile's visible keys and
// c = qk_scale * log2(e):
//   m_new = max(m, c * max_k s_k)       (= max_k of c * s_k: rounding is monotone)
//   alpha = 2^(m - m_new)               (0 while the row has seen no key)
//   P_k   = bf16(2^(fma(s_k, c, -m_new)))
//   l     = alpha * l + sum_k P_k,   acc = alpha * acc + V^T P
// where both sums run through the MFMA unit: l is the product of an all-ones
// A operand with the same P fragment, so it sums exactly the bf16 weights the
// PV product applies.  A masked score is -inf and gives P = 0; a row whose
// m_new is still -inf (no key seen yet) subtracts 0 instead, so no lane forms
// -inf - (-inf).
//
// KEEP = false drops the keep-state selects: a row with no visible key in the
// tile then has m_new == m, alpha == 1 (or 0 on a still-empty row) and P == 0,
// so m comes out bit-for-bit the same and l and acc gain only +-0 terms, which
// can change nothing but the sign of an exact-zero accumulator (l >= 0 sums
// +0 products and stays as it was); the merge adds such an accumulator into a
// sum that starts at +0 and stores -0 as +0, so every output bit is the same
// either way.  (Which form a kernel uses is measured: without the selects each
// PV product accumulates in place, while with them every product goes through
// a temporary that the next one waits for — a one-block tile at head dim 128
// computed alone takes 418 instead of 644 ns, two blocks 673 instead of 1192
// ns — but the four-block kernel then spills and the row-group kernel ran no
// faster.  The one-block split kernel takes them out and is held to two
// workgroups per compute unit at head dim <= 128, which it then fits in 256
// registers without spilling.)
//
// Two wave-uniform shortcuts leave every value bit-for-bit as computed in
// full: the key masks are applied only when some row of the wave does not see
// all 32 keys of the tile (a masked score is -inf, an unmasked one passes
// unchanged), and the accumulators are rescaled only when some row has a new
// maximum (otherwise alpha is exp2(0) = 1 exactly, or 0 on an accumulator
// that is still +0, so acc * alpha == acc).  Rescaling in place before the PV
// product equals scaling its input: a row without a visible key has
// m_new == m and keeps its accumulator either way.
template <int D, int QB, bool KEEP = true>
__device__ __forceinline__ void compute_tile(SplitState<D> (&st)[QB], const TileData<D>& t,
                                             const ItemLane<D> (&L)[QB], int tile, int g4, float qk_scale_log2) {
  constexpr int NSTEP = D / 32;
  constexpr int NBLK = D / 16;
  const int kb = tile << 5;
  bool inside = true;
#pragma unroll
  for (int b = 0; b < QB; ++b) inside &= L[b].rm.lo <= kb && kb + 31 <= L[b].rm.hi;
  const bool any_masked = __builtin_amdgcn_ballot_w64(!inside) != 0;
  // Raw scores: lane holds keys kb + 16h + 4*g4 + i (i = 0..3) of its row.
  float x[QB][2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    f32x4 sc[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) sc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
#pragma unroll
      for (int b = 0; b < QB; ++b) sc[b] = mfma16x16x32(__builtin_bit_cast(bf16x8, t.kf[h][s]), L[b].q[s], sc[b]);
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[b][h][i] = sc[b][i];
  }
  if (any_masked) {
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + 16 * h + 4 * g4 + i;
          if (key < L[b].rm.lo || key > L[b].rm.hi) x[b][h][i] = -INFINITY;
        }
  }
  float tmax[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    tmax[b] = x[b][0][0];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax[b] = fmaxf(tmax[b], x[b][h][i]);
  }
#pragma unroll
  for (int b = 0; b < QB; ++b) tmax[b] = row4_max(tmax[b]) * qk_scale_log2;

  bool live[QB];
  float m_new[QB], alpha[QB];
  bf16x8 pfrag[QB];
  bool rescale = false;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    live[b] = tmax[b] != -INFINITY;  // this row sees at least one key here
    m_new[b] = fmaxf(st[b].m, tmax[b]);
    alpha[b] = (st[b].m == -INFINITY) ? 0.f : exp2_hw(st[b].m - m_new[b]);
    rescale |= st[b].m != -INFINITY && m_new[b] != st[b].m;
    const float neg_m = m_new[b] == -INFINITY ? 0.f : -m_new[b];
    __bf16 pb[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[h][i] = (__bf16)exp2_hw(__builtin_fmaf(x[b][h][i], qk_scale_log2, neg_m));
    pfrag[b] = bf16x8{pb[0][0], pb[0][1], pb[0][2], pb[0][3], pb[1][0], pb[1][1], pb[1][2], pb[1][3]};
  }
  if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      st[b].lacc = st[b].lacc * alpha[b];
#pragma unroll
      for (int n = 0; n < NBLK; ++n) st[b].acc[n] = st[b].acc[n] * alpha[b];
    }
  }

#pragma unroll
  for (int n = 0; n < NBLK; ++n) {
    // De-interleave head-dim block n (e = n & 1) from the loaded pairs:
    // dword j of vf holds token j of rows e = 0 (low half) and e = 1 (high half).
    const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
    const u32x4 w0 = t.vf[0][n >> 1], w1 = t.vf[1][n >> 1];
    const u32x4 vv = {__builtin_amdgcn_perm(w0.y, w0.x, sel) & t.vmask[0].x,
                      __builtin_amdgcn_perm(w0.w, w0.z, sel) & t.vmask[0].y,
                      __builtin_amdgcn_perm(w1.y, w1.x, sel) & t.vmask[1].x,
                      __builtin_amdgcn_perm(w1.w, w1.z, sel) & t.vmask[1].y};
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const f32x4 res = mfma16x16x32(__builtin_bit_cast(bf16x8, vv), pfrag[b], st[b].acc[n]);
      st[b].acc[n] = (!KEEP || live[b]) ? res : st[b].acc[n];
    }
  }
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const f32x4 res = mfma16x16x32(__builtin_bit_cast(bf16x8, ones), pfrag[b], st[b].lacc);
    st[b].lacc = (!KEEP || live[b]) ? res : st[b].lacc;
    st[b].m = (!KEEP || live[b]) ? m_new[b] : st[b].m;
  }
}

// ---------------------------------------------------------------------------
// Work list.  An item is one (sequence, query-row block, KV head, split).  The
// plan kernel writes, for every sequence, the index of its first item
// (an exclusive prefix sum of integer counts, so exact whatever the order);
// item u of sequence s has local index l = u - first[s], with the KV head
// fastest (kvh = l % H_kv), then the split (lo_split(s) + (l / H_kv) %
// nsplit(s)), then the row block: neighbouring waves read the heads of the
// same physical pages together.
// A row block whose rows see no key of a split still owns that item; it is
// processed as one fully masked tile and writes nothing.
// ---------------------------------------------------------------------------
struct SeqSplits {
  int lo, n;  // first split meeting any row of the sequence, number of splits
};

// Splits are capped at ns, the workspace's splits per row (a length past the
// max_seq_len the call was sized for is a precondition violation; the cap keeps
// every partial store inside the row's ns slots, as the merge's cap keeps its
// loads, and the result is truncated there).
__device__ __forceinline__ SeqSplits seq_splits(int q_len, int k_len, int window, int S, int ns) {
  SeqSplits r{0, 0};
  if (q_len <= 0 || k_len <= 0 || q_len > k_len) return r;
  const int p_first = k_len - q_len;
  const int lo = window > 0 ? max(0, p_first - window + 1) : 0;
  r.lo = lo / S;
  r.n = min((k_len - 1) / S, ns - 1) - r.lo + 1;
  if (r.n <= 0) r = SeqSplits{0, 0};
  return r;
}

// Exclusive prefix sum of the per-sequence item counts over NT threads;
// store(i, v) receives plan[i] for i < num_seqs and the total at i = num_seqs.
template <int NT, typename Store>
__device__ __forceinline__ void plan_scan(const AttnSplitArgs& a, int* wave_tot, int* carry_sh, Store store) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int tq = (kRowsPerBlock >> a.log2_group) * a.qblocks;  // query tokens per work item
  if (tid == 0) *carry_sh = 0;
  __syncthreads();
  for (int base = 0; base < a.num_seqs; base += NT) {
    const int s = base + tid;
    int c = 0;
    if (s < a.num_seqs) {
      const int q_len = a.qsl[s + 1] - a.qsl[s];
      const SeqSplits sp = seq_splits(q_len, a.seq_lens[s], a.window, a.split, a.ns);
      c = sp.n > 0 ? ((q_len + tq - 1) / tq) * a.num_kv_heads * sp.n : 0;
    }
    int incl = c;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int before = *carry_sh;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    if (s < a.num_seqs) store(s, before + incl - c);
    __syncthreads();
    if (tid == NT - 1) *carry_sh = before + incl;
    __syncthreads();
  }
  if (tid == 0) store(a.num_seqs, *carry_sh);
}

__global__ __launch_bounds__(1024) void attn_plan_kernel(const AttnSplitArgs a) {
  __shared__ int wave_tot[16];
  __shared__ int carry_sh;
  plan_scan<1024>(a, wave_tot, &carry_sh, [&](int i, int v) { a.plan[i] = v; });
}

// Up to this many sequences, every workgroup of the split kernels computes the
// plan itself into LDS at its start (the scan costs each workgroup less than
// the separate launch it replaces); beyond it a one-workgroup launch writes the
// plan to the workspace first.
constexpr int kLdsPlanSeqs = 2048;

// Plan entry i (the first item of sequence i; the total at i = num_seqs), from
// the workgroup's LDS copy or from the workspace; wave-uniform.
struct PlanView {
  const int* lds;  // nullptr: the workspace copy a.plan
  int lds_asm;     // 1: the LDS copy is read by a load the compiler does not see
  __device__ __forceinline__ int at(const AttnSplitArgs& a, int i) const {
    if (lds && lds_asm) {
      // In a kernel with copies to LDS in flight the compiler orders every
      // LDS load after all of them; this table is written before the first
      // copy and never again, so it is read by a load of its own that waits
      // only for itself (and other LDS and scalar loads), in the same block.
      int v;
#if defined(__HIP_DEVICE_COMPILE__)
      const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int*)(lds + i);
      asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
#else
      v = lds[i];
#endif
      return __builtin_amdgcn_readfirstlane(v);
    }
    return lds ? __builtin_amdgcn_readfirstlane(lds[i]) : ldc(a.plan, i);
  }
};

// Wave-uniform description of one item.
struct Item {
  int valid;                 // 0: past the end of the work list
  int s, kvh, sigma, q0, tq0, nrow_tok, k_len, p_first;
  int tile_begin, tile_end;  // at least one tile
  int last_entry;            // last page-table entry the sequence uses
  const int32_t* pt_row;
};

// The item (sequence s, KV head kvh, split sigma, query tokens [tq0, tq0 + tq)
// of the sequence's q_len): its rows' positions and the tiles of the split
// that any of them sees.
__device__ __forceinline__ void fill_item(const AttnSplitArgs& a, Item& it, int s, int kvh, int sigma, int q0,
                                          int q_len, int k_len, int tq0, int tq) {
  it.s = s;
  it.kvh = kvh;
  it.sigma = sigma;
  it.q0 = q0;
  it.tq0 = tq0;
  it.nrow_tok = min(tq, q_len - it.tq0);
  it.k_len = k_len;
  it.p_first = k_len - q_len + it.tq0;
  const int p_last = it.p_first + it.nrow_tok - 1;
  const int lo_first = a.window > 0 ? max(0, it.p_first - a.window + 1) : 0;
  const int key_begin = max(sigma * a.split, lo_first);
  const int key_end = min(sigma * a.split + a.split, p_last + 1);
  it.tile_begin = key_begin < key_end ? (key_begin >> 5) : (sigma * a.split) >> 5;
  it.tile_end = key_begin < key_end ? ((key_end + 31) >> 5) : it.tile_begin + 1;
  it.last_entry = max(0, min((k_len + 15) / 16, a.pt_stride) - 1);
  it.pt_row = a.page_table + (int64_t)s * a.pt_stride;
}

__device__ __forceinline__ Item decode_item(const AttnSplitArgs& a, const PlanView& pv, int u, int total) {
  Item it;
  it.valid = u < total;
  it.s = 0; it.kvh = 0; it.sigma = 0; it.q0 = 0; it.tq0 = 0; it.nrow_tok = 0; it.k_len = 0; it.p_first = 0;
  it.tile_begin = 0; it.tile_end = 1; it.last_entry = 0; it.pt_row = a.page_table;
  if (!it.valid) return it;
  int lo = 0, hi = a.num_seqs - 1;  // largest s with plan[s] <= u
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pv.at(a, mid) <= u) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int local = u - pv.at(a, s);
  const int q0 = ldc(a.qsl, s);
  const int q_len = ldc(a.qsl, s + 1) - q0;
  const int k_len = ldc(a.seq_lens, s);
  const SeqSplits sp = seq_splits(q_len, k_len, a.window, a.split, a.ns);
  const int tq = (kRowsPerBlock >> a.log2_group) * a.qblocks;
  const int kvh = local % a.num_kv_heads;
  const int rest = local / a.num_kv_heads;
  fill_item(a, it, s, kvh, sp.lo + rest % sp.n, q0, q_len, k_len, (rest / sp.n) * tq, tq);
  return it;
}

// This lane's query row in block blk of an item (token t of the item, head hh
// of the GQA group).
template <int D>
__device__ __forceinline__ ItemLane<D> item_lane(const AttnSplitArgs& a, const Item& it, int lane, int blk) {
  constexpr int NSTEP = D / 32;
  const int r = lane & 15, g4 = lane >> 4;
  const int t = blk * (kRowsPerBlock >> a.log2_group) + (r >> a.log2_group);
  const int hh = r & ((1 << a.log2_group) - 1);
  const bool row_ok = it.valid && (t < it.nrow_tok) && (it.q0 + it.tq0 + t < a.num_tokens);
  const int p = it.p_first + t;
  ItemLane<D> L;
  const int split_lo = it.sigma * a.split;
  L.rm.lo = max(a.window > 0 ? max(0, p - a.window + 1) : 0, split_lo);
  L.rm.hi = min(p, split_lo + a.split - 1);
  if (!row_ok || p < 0) { L.rm.lo = 1; L.rm.hi = 0; }
  // Rows past the item (padding columns of the MFMA) read the item's first
  // row instead: their mask is empty, so their scores never reach any result
  // (each MFMA output column depends only on its own Q column).
  const int tok = min(it.q0 + it.tq0 + (row_ok ? t : 0), max(a.num_tokens - 1, 0));
  const uint16_t* qrow = a.q + (int64_t)tok * a.q_stride + (int64_t)((it.kvh << a.log2_group) + hh) * D;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st)
    L.q[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + (4 * st + g4) * 8));
  return L;
}

// Cache policy of the partial stores: device scope (sc1).  Measured against
// non-temporal stores on the 8B-shaped decode at batch 256: the split phase
// 788 -> 762 us and the merge, which reads the partials back, 19 -> 14 us.
constexpr int kPartialStore = 16;

template <int D>
__device__ __forceinline__ void write_partial(const AttnSplitArgs& a, const Item& it, const ItemLane<D>& L,
                                              const SplitState<D>& st, int lane, int blk) {
  if (L.rm.lo > L.rm.hi) return;
  const int r = lane & 15, g4 = lane >> 4;
  const int tb = blk * (kRowsPerBlock >> a.log2_group);  // first token of the block within the item
  const int t = r >> a.log2_group;                       // this lane's token within the block
  const int hh = r & ((1 << a.log2_group) - 1);
  // Partial (row, split) index of the block's first row; this lane's row is
  // rel further (rows are num_q_heads apart per token, ns splits per row).
  // The resources are uniform across the wave; offsets fit in 32 bits
  // (16 * H_q * ns * D * 4 < 2^31, checked on the host).
  const int64_t idx0 =
      ((int64_t)(it.q0 + it.tq0 + tb) * a.num_q_heads + (it.kvh << a.log2_group)) * a.ns + it.sigma;
  const uint32_t rel = (uint32_t)((t * a.num_q_heads + hh) * a.ns);
  const __amdgpu_buffer_rsrc_t mr =
      __builtin_amdgcn_make_buffer_rsrc(a.ws_ml + idx0, (short)0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc(a.ws_acc + idx0 * D, (short)0, 0x7fffffff, 0x00020000);
  if (g4 == 0)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(st.m), __float_as_uint(st.l())}, mr, (int)(rel * 8u), 0,
                                          kPartialStore);
  // Column blocks n and n + 1 in one 16-byte store per lane: lane rows g4 and
  // g4 ^ 1 (lanes 16 apart) trade halves, so that an even row holds head dims
  // 16n + 4g4 .. + 7 of block n (its own four, then its partner's) and an odd
  // row 16(n+1) + 4(g4-1) .. + 7 of block n + 1 (its partner's four, then its
  // own).  The swap moves odd rows of its first operand and even rows of its
  // second; either way a lane's words come out as (first, second).
  const bool odd = (g4 & 1) != 0;
#pragma unroll
  for (int n = 0; n < D / 16; n += 2) {
    const u32x2 x = acc_to_bf16(st.acc[n]), y = acc_to_bf16(st.acc[n + 1]);
    const auto w0 = __builtin_amdgcn_permlane16_swap(x.x, y.x, false, false);
    const auto w1 = __builtin_amdgcn_permlane16_swap(x.y, y.y, false, false);
    const u32x4 v = {w0[0], w1[0], w0[1], w1[1]};
    const uint32_t d0 = odd ? 16 * (n + 1) + 4 * (g4 - 1) : 16 * n + 4 * g4;
    __builtin_amdgcn_raw_buffer_store_b128(v, ar, (int)((rel * D + d0) * 2u), 0, kPartialStore);
  }
}

// ---------------------------------------------------------------------------
// Split phase, persistent: the grid holds as many waves as the GPU keeps
// resident; wave w processes items w, w + W, w + 2W, ...  Tiles stream through
// two register buffers: while tile k is computed, tile k+1 is loading, and
// tile k+1 may already belong to the wave's next item (whose description is
// decoded while the current item is computed).  Which wave
// computes an item, and when, has no effect on its arithmetic.
//
// An item holds QB query-row blocks (QB = 1 for decode-shaped batches, more
// for prefill-shaped ones, where a loaded K/V tile then serves QB blocks).
// Every block runs compute_tile exactly as it would alone: the same tile, the
// same instructions, its own state.  The item's tile range is the union of its
// blocks' ranges, and a tile outside a row's range leaves that row's state
// unchanged, so the choice of QB never changes a bit of any row.
// ---------------------------------------------------------------------------
template <int D, int QB>
struct SplitWave {
  const AttnSplitArgs& a;
  PlanView pv;
  int lane, g4, total, stride, u;
  Item cur, nxt;
  ItemLane<D> curL[QB];
  SplitState<D> st[QB];
  int ct;  // tile of `cur` being computed

  __device__ __forceinline__ void begin_item() {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      curL[b] = item_lane<D>(a, cur, lane, b);
      st[b].init();
    }
  }

  // Compute tile `ct` of `cur` from Bc while the next tile of the stream loads
  // into Bl.  Returns false once the wave has no item left.
  __device__ __forceinline__ bool step(TileData<D>& Bc, TileData<D>& Bl) {
    const bool in_cur = ct + 1 < cur.tile_end;
    const Item& L = in_cur ? cur : nxt;
    const int lt = in_cur ? ct + 1 : nxt.tile_begin;
    const int lend = (in_cur || nxt.valid) ? L.tile_end : lt;  // dead load past the last item
    load_tile(a, L.kvh, L.k_len, lt, lend, tile_pages(L.pt_row, L.last_entry, lt), lane, Bl);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile<D, QB, (QB > 1)>(st, Bc, curL, ct, g4, a.qk_scale_log2);
    __builtin_amdgcn_sched_barrier(0);
    if (in_cur) {
      ++ct;
      return true;
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) write_partial(a, cur, curL[b], st[b], lane, b);
    if (!nxt.valid) return false;
    cur = nxt;
    begin_item();  // Q loads overlap the tile loads already in flight
    u += stride;
    ct = cur.tile_begin;
    nxt = decode_item(a, pv, u + stride, total);
    return true;
  }
};

template <int D, int QB>
__global__ __launch_bounds__(64 * kSplitWaves, (QB == 1 && D <= 128) ? 2 : 1) void attn_split_kernel(const AttnSplitArgs a) {
  const int lane = threadIdx.x & 63;
  // Wave index, made visibly wave-uniform so everything derived from the
  // item index stays in scalar registers (scalar page-table loads).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __shared__ int plan_s[kLdsPlanSeqs + 1];
  __shared__ int wave_tot[kSplitWaves];
  __shared__ int carry_sh;
  SplitWave<D, QB> w{a};
  w.pv.lds = nullptr;
  w.pv.lds_asm = 0;
  if (a.num_seqs <= kLdsPlanSeqs) {
    plan_scan<64 * kSplitWaves>(a, wave_tot, &carry_sh, [&](int i, int v) { plan_s[i] = v; });
    __syncthreads();
    w.pv.lds = plan_s;
  }
  w.lane = lane;
  w.g4 = lane >> 4;
  w.total = w.pv.at(a, a.num_seqs);
  w.stride = gridDim.x * kSplitWaves;
  // Item u of the first round goes to wave u % kSplitWaves of workgroup
  // u / kSplitWaves, or, when there are fewer items than waves (spread), to
  // rank u / gridDim.x of workgroup u % gridDim.x, so that a small batch's
  // items run on as many compute units as possible.  Ranks take the waves in
  // order, rotated by two in the upper half of the grid: the two workgroups a
  // compute unit holds then start their first items on different SIMDs.
  const int G = (int)gridDim.x;
  const int rank = (wave + kSplitWaves - ((int)blockIdx.x >= G / 2 ? 2 : 0)) % kSplitWaves;
  w.u = a.spread ? rank * G + (int)blockIdx.x : (int)blockIdx.x * kSplitWaves + wave;
  w.cur = decode_item(a, w.pv, w.u, w.total);
  if (!w.cur.valid) return;
  w.begin_item();
  w.nxt = decode_item(a, w.pv, w.u + w.stride, w.total);
  w.ct = w.cur.tile_begin;
  TileData<D> buf0, buf1;
  load_tile(a, w.cur.kvh, w.cur.k_len, w.ct, w.cur.tile_end, tile_pages(w.cur.pt_row, w.cur.last_entry, w.ct),
            lane, buf0);
  while (w.step(buf0, buf1) && w.step(buf1, buf0)) {
  }
}

// ---------------------------------------------------------------------------
// Split phase for prefill-shaped batches: workgroup-shared K/V tiles.  A work
// item holds kSharedBlocks query-row blocks of one (sequence, KV head, split);
// each of the four waves owns two of them.  The K/V tiles of the item stream
// through an R-slot LDS ring (buffer loads straight to LDS, 1 KiB per
// instruction, every wave copying a quarter of each tile), and every wave
// reads each tile from LDS into exactly the registers load_tile fills and
// runs the same compute_tile on its two blocks: the arithmetic of every row is
// the one-block arithmetic, so every bit of its partials is the same.  One
// copy of a tile feeds eight blocks, and the per-wave state (two blocks, one
// tile) leaves room for two waves per SIMD.
//
// Per step i (all four waves walk the same stream of tiles):
//   issue this wave's chunks of tile i + PD into slot (i + PD) % R, wait for
//   this wave's chunks of tile i;  barrier;  read slot i % R into registers;
//   compute tile i for the wave's two blocks (and write their partials at an
//   item's last tile).
// Slot (i + PD) % R last held tile i + PD - R <= i - 2, which every wave read
// before it reached the barrier of step i - 1: one barrier per step suffices.
// Each wave issues the same number of copies every step (tiles past the end
// of the stream copy nothing, through an empty resource), so its wait count
// is fixed; loads and stores it issues besides only make that wait stronger.
// ---------------------------------------------------------------------------
constexpr int kSharedWaves = 4;
constexpr int kSharedBlocks = 8;  // query-row blocks per item: two per wave

template <int D>
struct SharedShape {
  static constexpr int KCH = D / 32;       // 1 KiB chunks per K (or V) page of one KV head
  static constexpr int NCH = 4 * KCH;      // chunks per tile: K page 0, K page 1, V page 0, V page 1
  static constexpr int TILE = NCH * 1024;  // bytes per ring slot
  static constexpr int R = 4;              // ring slots
  static constexpr int PD = 2;             // tiles loading ahead of the one computed
  static_assert(R - PD >= 2, "a refilled slot was read two steps earlier: one barrier per step orders it");
  static constexpr int CPW = NCH / kSharedWaves;  // chunks per wave per tile
  static_assert(NCH % kSharedWaves == 0, "chunks split evenly over the waves");
};

typedef __attribute__((address_space(3))) void lds_void_t;

template <int n>
__device__ __forceinline__ void shared_wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

__device__ __forceinline__ u32x4 shared_lds_read(uint32_t addr) {
  u32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
#else
  v = u32x4{addr, 0u, 0u, 0u};
#endif
  return v;
}

// Cursor over one workgroup's tile stream: items u, u + G, ... and their tiles.
struct TileCursor {
  Item it;
  int u, t;
  __device__ __forceinline__ void start(const AttnSplitArgs& a, const PlanView& pv, int u0, int total) {
    u = u0;
    it = decode_item(a, pv, u, total);
    t = it.tile_begin;
  }
  // Moves to the next tile; true when that ended the item.
  __device__ __forceinline__ bool advance(const AttnSplitArgs& a, const PlanView& pv, int stride, int total) {
    if (++t < it.tile_end) return false;
    u += stride;
    it = decode_item(a, pv, u, total);
    t = it.tile_begin;
    return true;
  }
};

// This wave's chunks (w, w + 4, ...) of the cursor's tile into ring slot `slot`,
// through the page resources load_tile would use.  Chunk j of a tile is KiB
// j % KCH of page j / KCH (K page 0, K page 1, V page 0, V page 1).  The
// resources are named, not an array: an array indexed by the wave number
// would leave the scalar registers, and every copy would then be issued
// through a loop that reads the resource back one lane at a time.
template <int D>
__device__ __forceinline__ void shared_issue(const AttnSplitArgs& a, const TileCursor& lc, char* ring, int slot,
                                             int w, int lane) {
  using S = SharedShape<D>;
  constexpr int PAGE_BYTES = D * 16 * 2;
  const int64_t head_elems = (int64_t)D * 16;
  const int2 pid = tile_pages(lc.it.pt_row, lc.it.last_entry, lc.t);
  __amdgpu_buffer_rsrc_t rk0, rk1, rv0, rv1;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int entry = 2 * lc.t + b;
    const int raw = b == 0 ? pid.x : pid.y;
    const int pgc = min(max(raw, 0), a.num_pages - 1);
    const bool ok = lc.it.valid && lc.t < lc.it.tile_end && entry * 16 < lc.it.k_len && entry < a.pt_stride &&
                    raw == pgc;
    const int64_t base = ((int64_t)pgc * a.num_kv_heads + lc.it.kvh) * head_elems;
    const __amdgpu_buffer_rsrc_t kr = page_rsrc(a.k_cache + base, ok ? PAGE_BYTES : 0);
    const __amdgpu_buffer_rsrc_t vr = page_rsrc(a.v_cache + base, ok ? PAGE_BYTES : 0);
    if (b == 0) {
      rk0 = kr;
      rv0 = vr;
    } else {
      rk1 = kr;
      rv1 = vr;
    }
  }
#pragma unroll
  for (int k = 0; k < S::CPW; ++k) {
    const int j = w + kSharedWaves * k;  // chunk of the tile
    // Page of the chunk: a constant when a page holds a multiple of four
    // chunks (w < 4 stays inside one page), else chosen by a uniform select.
    const int page = S::KCH % kSharedWaves == 0 ? (kSharedWaves * k) / S::KCH : j / S::KCH;
    const __amdgpu_buffer_rsrc_t rs = page == 0 ? rk0 : (page == 1 ? rk1 : (page == 2 ? rv0 : rv1));
    lds_void_t* dst = (lds_void_t*)(ring + slot * S::TILE + j * 1024);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, (j % S::KCH) * 1024 + lane * 16, 0, 0, kStreamLoad);
  }
}

// The tile in the ring slot at slot_addr into the registers load_tile fills,
// plus the V zero-fill masks load_tile records.
template <int D>
__device__ __forceinline__ void shared_read_tile(const AttnSplitArgs& a, const TileCursor& cc, uint32_t slot_addr,
                                                 int lane, TileData<D>& t) {
  using S = SharedShape<D>;
  const int r = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int st = 0; st < S::KCH; ++st)
      t.kf[b][st] = shared_lds_read(slot_addr + (b * S::KCH + st) * 1024 + lane * 16);
#pragma unroll
    for (int np = 0; np < S::KCH; ++np)
      t.vf[b][np] = shared_lds_read(slot_addr + ((2 + b) * S::KCH + np) * 1024 + r * 64 + g4 * 16);
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int k = 0; k < S::KCH; ++k) {
      asm volatile("" : "+v"(t.kf[b][k]));
      asm volatile("" : "+v"(t.vf[b][k]));
    }
#endif
  const int2 pid = tile_pages(cc.it.pt_row, cc.it.last_entry, cc.t);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int entry = 2 * cc.t + b;
    const int raw = b == 0 ? pid.x : pid.y;
    const int pgc = min(max(raw, 0), a.num_pages - 1);
    const bool ok = entry * 16 < cc.it.k_len && entry < a.pt_stride && raw == pgc;
    const int nl = min(16, cc.it.k_len - (cc.t * 32 + 16 * b)) - 4 * g4;  // valid keys among this lane's four
    t.vmask[b].x = !ok ? 0u : (nl >= 2 ? 0xffffffffu : (nl == 1 ? 0x0000ffffu : 0u));
    t.vmask[b].y = !ok ? 0u : (nl >= 4 ? 0xffffffffu : (nl == 3 ? 0x0000ffffu : 0u));
  }
}

template <int D>
__global__ __launch_bounds__(64 * kSharedWaves, 2) void attn_split_shared_kernel(const AttnSplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using S = SharedShape<D>;
  __shared__ __attribute__((aligned(1024))) char ring[S::R * S::TILE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The plan: up to kLdsPlanSeqs sequences every workgroup computes it into
  // LDS before its first copy (read back with loads of their own, see
  // PlanView), beyond that it comes from the workspace (scalar loads).
  __shared__ int plan_s[kLdsPlanSeqs + 1];
  __shared__ int wave_tot[kSharedWaves];
  __shared__ int carry_sh;
  PlanView pv;
  pv.lds = nullptr;
  pv.lds_asm = 0;
  if (a.num_seqs <= kLdsPlanSeqs) {
    plan_scan<64 * kSharedWaves>(a, wave_tot, &carry_sh, [&](int i, int v) { plan_s[i] = v; });
    __syncthreads();
    pv.lds = plan_s;
    pv.lds_asm = 1;
  }
  const int total = pv.at(a, a.num_seqs);
  const int G = (int)gridDim.x;
  TileCursor cc, lc;
  cc.start(a, pv, (int)blockIdx.x, total);
  if (!cc.it.valid) return;  // the whole workgroup: the item index depends on blockIdx only
  lc = cc;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)(lds_void_t*)ring;
  for (int p = 0; p < S::PD; ++p) {  // tiles 0 .. PD - 1 into slots 0 .. PD - 1
    shared_issue<D>(a, lc, ring, p, wave, lane);
    lc.advance(a, pv, G, total);
  }
  SplitState<D> st[2];
  ItemLane<D> L[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    L[b] = item_lane<D>(a, cc.it, lane, 2 * wave + b);
    st[b].init();
  }
  TileData<D> td;
  int slot = 0;  // ring slot of step i (i % R)
  for (;;) {
    shared_issue<D>(a, lc, ring, (slot + S::PD) % S::R, wave, lane);
    shared_wait_vm<S::PD * S::CPW>();  // the chunks of the PD later tiles may still fly
    lc.advance(a, pv, G, total);
    __builtin_amdgcn_s_barrier();  // tile i is in slot `slot`
    shared_read_tile<D>(a, cc, ring_addr + slot * S::TILE, lane, td);
    compute_tile<D, 2, false>(st, td, L, cc.t, lane >> 4, a.qk_scale_log2);
    const Item done = cc.it;
    if (cc.advance(a, pv, G, total)) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        write_partial(a, done, L[b], st[b], lane, 2 * wave + b);
        L[b] = item_lane<D>(a, cc.it, lane, 2 * wave + b);
        st[b].init();
      }
      if (!cc.it.valid) break;
    }
    slot = slot + 1 == S::R ? 0 : slot + 1;
  }
  shared_wait_vm<0>();  // no copy outlives the workgroup's LDS
#endif
}

// ---------------------------------------------------------------------------
// Merge arithmetic of one row's four head-dim values, shared by the merge
// kernel and the row-group decode kernel so that both give the same bits:
// after m* = max_s m_s (exact in any order), splits are folded in increasing
// order, w = 2^(m_s - m*), L += w l_s, N += w acc_s (one fma each); then
// o = N / L, -0 stored as +0, rounded to bf16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void merge_fold(float mstar, float2 ml, const f32x4& acc, float& L, f32x4& N) {
  const float w = exp2_hw(ml.x - mstar);
  L = __builtin_fmaf(w, ml.y, L);
#pragma unroll
  for (int i = 0; i < 4; ++i) N[i] = __builtin_fmaf(w, acc[i], N[i]);
}

__device__ __forceinline__ u32x2 merge_finish(const f32x4& N, float L) {
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (__bf16)(N[i] / L + 0.0f);
  return __builtin_bit_cast(u32x2, o);
}

// ---------------------------------------------------------------------------
// Merge phase: one thread per (row, 4 head-dim elements).  Splits are combined
// in increasing order: m* = max m_s, w_s = 2^(m_s - m*), L = sum w_s l_s,
// N = sum w_s acc_s, o = N / L.  With a single split w = 1 exactly and the
// result is acc / l.
//
// Each wave serves one query token (all its rows share the split range), so
// the sequence lookup and the split bounds are wave-uniform and go through
// the scalar unit; a token's H_q rows take ceil(H_q * D / 256) waves.  Up to
// kOnePass splits every load of a row is issued before any is used (one
// round trip); beyond that the maxima come first, then the sums in groups.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnMergeArgs a) {
  constexpr int TPR = D / 4;
  const int wpt = (a.num_q_heads * TPR + 63) / 64;  // waves per token
  const int gw = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int tok = __builtin_amdgcn_readfirstlane(gw / wpt);
  if (tok >= a.num_tokens) return;
  const int idx = (gw - tok * wpt) * 64 + (int)(threadIdx.x & 63);
  const int h = idx / TPR, dq = idx % TPR;
  if (h >= a.num_q_heads) return;
  // Largest s with qsl[s] <= tok (every sequence has a query row).
  int s = 0;
  if (a.num_tokens == a.num_seqs) {
    s = tok;
  } else {
    int hi = a.num_seqs - 1;
    while (s < hi) {
      const int mid = (s + hi + 1) >> 1;
      if (ldc(a.qsl, mid) <= tok) s = mid; else hi = mid - 1;
    }
  }
  const int q0 = ldc(a.qsl, s);
  const int q_len = ldc(a.qsl, s + 1) - q0;
  const int k_len = ldc(a.seq_lens, s);
  const int p = k_len - q_len + (tok - q0);
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int sig_lo = lo / a.split;
  const int sig_hi = min(p / a.split, a.ns - 1);
  const int64_t row = (int64_t)tok * a.num_q_heads + h;
  uint16_t* op = a.out + row * D + 4 * dq;
  if (p < 0 || sig_lo > sig_hi) {
    *reinterpret_cast<u32x2*>(op) = u32x2{0u, 0u};
    return;
  }
  const float2* ml = a.ws_ml + row * a.ns;
  const uint16_t* ap = a.ws_acc + row * a.ns * D + 4 * dq;
  const int nsp = sig_hi - sig_lo + 1;
  constexpr int kOnePass = 16, kMaxGroup = 32, kSumGroup = 16;
  float L = 0.f;
  f32x4 N = {0.f, 0.f, 0.f, 0.f};
  if (nsp <= kOnePass) {
    float2 v[kOnePass];
    u32x2 av[kOnePass];
#pragma unroll
    for (int j = 0; j < kOnePass; ++j) {
      if (j < nsp) {
        v[j] = ml[sig_lo + j];
        av[j] = *reinterpret_cast<const u32x2*>(ap + (int64_t)(sig_lo + j) * D);
      }
    }
    float mstar = -INFINITY;
#pragma unroll
    for (int j = 0; j < kOnePass; ++j)
      if (j < nsp) mstar = fmaxf(mstar, v[j].x);
#pragma unroll
    for (int j = 0; j < kOnePass; ++j)
      if (j < nsp) merge_fold(mstar, v[j], bf16_to_acc(av[j]), L, N);
    *reinterpret_cast<u32x2*>(op) = merge_finish(N, L);
    return;
  }
  // The maximum: up to 32 splits' m loaded together per round (max is exact in
  // any order, so the grouping changes no bit).
  float mstar = -INFINITY;
  for (int base = sig_lo; base <= sig_hi; base += kMaxGroup) {
    float mv[kMaxGroup];
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j) mv[j] = base + j <= sig_hi ? ml[base + j].x : -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j) mstar = fmaxf(mstar, mv[j]);
  }
  // The sums, in increasing split order; the loads of up to 16 splits are
  // issued before any of them is accumulated.
  for (int base = sig_lo; base <= sig_hi; base += kSumGroup) {
    float2 v[kSumGroup];
    u32x2 av[kSumGroup];
#pragma unroll
    for (int j = 0; j < kSumGroup; ++j) {
      if (base + j <= sig_hi) {
        v[j] = ml[base + j];
        av[j] = *reinterpret_cast<const u32x2*>(ap + (int64_t)(base + j) * D);
      }
    }
#pragma unroll
    for (int j = 0; j < kSumGroup; ++j)
      if (base + j <= sig_hi) merge_fold(mstar, v[j], bf16_to_acc(av[j]), L, N);
  }
  *reinterpret_cast<u32x2*>(op) = merge_finish(N, L);
}

// ---------------------------------------------------------------------------
// Decode, row-group mapping: split and merge in one launch, partials in LDS.
//
// A row group is one (sequence, KV head) of a decode batch: the G query heads
// that read that KV head, one row each.  Its tasks are its splits, and a task
// is exactly a work item of the split kernel (the same tile range, load_tile,
// compute_tile, one query-row block), so each split's (m, l, acc) has the same
// bits.  The partial goes to an LDS ring instead of the workspace, and the wave
// that completes a row group's last split folds its partials with the merge
// kernel's arithmetic (merge_fold, merge_finish, splits in increasing order)
// and writes the G output rows: the output is bitwise that of split + merge.
//
// Work distribution (it changes no bit).  A one-workgroup plan launch ranks
// the sequences by visible keys, most first (ties by index), into the
// workspace plan and zeroes a claim counter after it.  Position r of that
// order is the row group (sequence order[r / H_kv], KV head r % H_kv).  The
// row-group kernel runs one workgroup per CU (W workgroups; eight waves, four
// at head dim 256).
// The first rg_static_rounds * W positions are dealt in a snake (round i gives
// workgroup g position i W + g in even rounds, i W + W - 1 - g in odd ones),
// so every workgroup starts with a similar total; the rest, the smallest row
// groups, are taken one at a time from the shared counter by whichever
// workgroup runs out of tasks first, which evens out compute units that run
// at different speeds.  Inside a workgroup the tasks are handed out one at a
// time under an LDS lock: the splits of the current row group in order, then
// those of the next.  A wave takes its next task one tile before its current
// task's last tile is loaded (so the next task's first tile loads while that
// last tile is computed) and not earlier, so that when the work runs out no
// wave holds more than about one task.
//
// Ring protocol.  The workgroup's task j writes its partial to ring entry
// j mod C once gen[j mod C] == j / C, i.e. once the row group of task j - C
// has been merged; a merge raises the generation of the entries it read.  A
// row group's tasks are consecutive, tasks are handed out in increasing j, and
// the launcher takes this mapping only when every row group has at most C
// splits, so every task a waiting wave depends on precedes its own and is held
// by a wave that is not waiting: each wait ends.  Each is bounded all the same
// (a wrong count ends the wait instead of hanging the kernel).
// ---------------------------------------------------------------------------
// Waves per workgroup: two per SIMD where the split state allows it (head
// dim <= 128), one at head dim 256.
template <int D>
constexpr int rg_waves() { return D <= 128 ? 8 : 4; }
constexpr int kRgMaxSeqs = 2048;        // sequences the plan launch ranks (in LDS)
constexpr int kRgRingBytes = 120 * 1024;
constexpr int kRgMaxEntries = 224;      // ring entries; unmerged row groups < kRgSlots
constexpr int kRgSlots = 256;           // row-group descriptors (a ring)
// Polls of a ring entry or of the lock (each after a short sleep): about a
// millisecond, far beyond any legitimate wait.  After one wait has run out the
// workgroup stops waiting altogether, so a broken count costs at most that once.
constexpr int kRgSpinLimit = 1 << 14;

// Ring entry of one task: acc bf16 [G][D] (rounded as for the workspace), then
// (m, l) float2 [G]; 16-byte multiple.
__host__ __device__ inline int rg_entry_bytes(int D, int G) { return (G * (2 * D + 8) + 15) & ~15; }
__host__ __device__ inline int rg_entries(int D, int G) {
  const int c = kRgRingBytes / rg_entry_bytes(D, G);
  return c < kRgMaxEntries ? c : kRgMaxEntries;
}

// Visible keys of a decode row of length k_len (0 for a row that is not a
// valid decode row).
__device__ __forceinline__ int rg_visible(const AttnSplitArgs& a, int s) {
  const int q0 = a.qsl[s], q_len = a.qsl[s + 1] - q0, k_len = a.seq_lens[s];
  if (q_len != 1 || k_len < 1) return 0;
  return k_len - (a.window > 0 ? max(0, k_len - a.window) : 0);
}

// Plan: plan[r] = the sequence of rank r (most visible keys first, ties by
// index) for r < num_seqs, and plan[num_seqs] = 0, the row-group claim counter.
// A sequence's rank counts the sequences ahead of it; P = 1024 / B' threads
// (B' = num_seqs rounded up to a power of two, P <= 64) share that count, each
// over a 1/P slice of the keys read four at a time, and sum it in a fixed
// xor tree.
__global__ __launch_bounds__(1024) void attn_rowgroup_plan_kernel(const AttnSplitArgs a) {
  __shared__ __attribute__((aligned(16))) int key[kRgMaxSeqs];
  const int B = a.num_seqs, tid = threadIdx.x;
  const int B4 = (B + 3) & ~3;
  for (int s = tid; s < B4; s += 1024) key[s] = s < B ? rg_visible(a, s) : -1;
  __syncthreads();
  int bp = 1;
  while (bp < B) bp <<= 1;
  const int P = bp >= 1024 ? 1 : min(64, 1024 / bp);  // threads per sequence, a power of two
  const int part = tid & (P - 1);
  const int quads = B4 >> 2;
  const int q_lo = part * quads / P, q_hi = (part + 1) * quads / P;
  for (int s0 = tid / P; s0 < bp; s0 += 1024 / P) {
    const int s = s0;  // every thread of a group runs the same iterations (the shuffles below need all of them)
    const int v = s < B ? key[s] : 0;
    int r = 0;
    for (int q = q_lo; q < q_hi; ++q) {
      const int4 w = *reinterpret_cast<const int4*>(key + 4 * q);
      const int t = 4 * q;
      r += (w.x > v) | ((w.x == v) & (t < s));
      r += (w.y > v) | ((w.y == v) & (t + 1 < s));
      r += (w.z > v) | ((w.z == v) & (t + 2 < s));
      r += (w.w > v) | ((w.w == v) & (t + 3 < s));
    }
    for (int off = 1; off < P; off <<= 1) r += __shfl_xor(r, off);
    if (part == 0 && s < B) a.plan[r] = s;
  }
  if (tid == 0) a.plan[B] = 0;
}

struct RgDesc {
  int s, kvh, lo, q0, first, n;  // sequence, KV head, first split, output token, first task, splits
};

struct RgShared {
  RgDesc g[kRgSlots];             // row group k at slot k % kRgSlots
  int g_done[kRgSlots];           // tasks of the row group whose partial is in the ring
  int gen[kRgMaxEntries];         // ring entry generations
  int lock;                       // task hand-out
  int next_task, cur_k, cur_i, started, exhausted, static_round;
  int broken;                     // set when a wait ran out: no wait is made after it
};

__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// One task as handed out (wave-uniform): task index j, row group k, split sigma.
struct RgTask {
  int j, k, sigma;
};

template <int D>
struct RgWave {
  const AttnSplitArgs& a;
  RgShared& sh;
  char* ring;
  int lane, g4, G, C, EB;
  RgTask tc, tn;  // tasks of cur and nxt
  bool have_nxt;  // nxt has been claimed
  Item cur, nxt;
  ItemLane<D> curL[1];
  SplitState<D> st[1];
  int ct;

  __device__ __forceinline__ bool broken() const {
    return rfl(__hip_atomic_load(&sh.broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0;
  }

  // A row group with no visible key (a length of 0, or past the splits the
  // call was sized for) is written as zeros, as the merge kernel does.
  __device__ __forceinline__ void zero_rows(int q0, int kvh) const {
    uint16_t* op = a.out + ((int64_t)q0 * a.num_q_heads + (kvh << a.log2_group)) * D;
    for (int i = 0; i < (G * D) / 4; ++i) *reinterpret_cast<u32x2*>(op + 4 * i) = u32x2{0u, 0u};
  }

  // Next task of the workgroup (lane 0 under the lock; j < 0: none left).
  __device__ __forceinline__ RgTask claim() {
    RgTask t{-1, 0, 0};
    if (lane == 0) {
      int spins = 0;
      for (;;) {
        int expected = 0;
        if (__hip_atomic_compare_exchange_strong(&sh.lock, &expected, 1, __ATOMIC_ACQUIRE, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP))
          break;
        if (++spins == kRgSpinLimit || __hip_atomic_load(&sh.broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
          __hip_atomic_store(&sh.broken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      int k = sh.cur_k, i = sh.cur_i;
      bool have = k >= 0 && i < sh.g[k % kRgSlots].n;
      while (!have && !sh.exhausted) {
        const int R = a.num_seqs * a.num_kv_heads;
        const int W = (int)gridDim.x;
        int r;
        if (sh.static_round < a.rg_static_rounds) {
          const int i = sh.static_round++;
          r = i * W + ((i & 1) ? W - 1 - (int)blockIdx.x : (int)blockIdx.x);
          if (r >= R) continue;
        } else {
          r = a.rg_static_rounds * W +
              __hip_atomic_fetch_add(a.plan + a.num_seqs, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (r >= R) {
          sh.exhausted = 1;
          break;
        }
        const int s = a.plan[r / a.num_kv_heads];
        const int kvh = r % a.num_kv_heads;
        const int q0 = a.qsl[s], q_len = a.qsl[s + 1] - q0;
        const bool ok = q_len == 1 && q0 >= 0 && q0 < a.num_tokens && s >= 0 && s < a.num_seqs;
        const SeqSplits sp = ok ? seq_splits(1, a.seq_lens[s], a.window, a.split, a.ns) : SeqSplits{0, 0};
        if (sp.n <= 0) {
          if (ok) zero_rows(q0, kvh);
          continue;
        }
        k = sh.started++;
        RgDesc& d = sh.g[k % kRgSlots];
        d.s = s;
        d.kvh = kvh;
        d.lo = sp.lo;
        d.q0 = q0;
        d.first = sh.next_task;
        d.n = sp.n;
        sh.g_done[k % kRgSlots] = 0;
        sh.cur_k = k;
        i = 0;
        have = true;
      }
      if (have) {
        t = RgTask{sh.next_task++, k, sh.g[k % kRgSlots].lo + i};
        sh.cur_i = i + 1;
      }
      __hip_atomic_store(&sh.lock, 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    return RgTask{rfl(t.j), rfl(t.k), rfl(t.sigma)};
  }

  __device__ __forceinline__ Item task_item(const RgTask& t) const {
    Item it;
    it.valid = t.j >= 0;
    it.s = 0; it.kvh = 0; it.sigma = 0; it.q0 = 0; it.tq0 = 0; it.nrow_tok = 0; it.k_len = 0; it.p_first = 0;
    it.tile_begin = 0; it.tile_end = 1; it.last_entry = 0; it.pt_row = a.page_table;
    if (!it.valid) return it;
    const RgDesc& d = sh.g[t.k % kRgSlots];
    const int s = rfl(d.s);
    fill_item(a, it, s, rfl(d.kvh), t.sigma, rfl(d.q0), 1, ldc(a.seq_lens, s), 0, kRowsPerBlock >> a.log2_group);
    return it;
  }

  __device__ __forceinline__ void begin_item() {
    curL[0] = item_lane<D>(a, cur, lane, 0);
    st[0].init();
  }

  // Fold the n partials of row group k (ring entries of its tasks first ...
  // first + n - 1) in split order, write its G output rows, free the entries.
  __device__ __forceinline__ void merge_group(int k) {
    constexpr int QPR = D / 4;
    const RgDesc& d = sh.g[k % kRgSlots];
    const int f = rfl(d.first), n = rfl(d.n), kvh = rfl(d.kvh), q0 = rfl(d.q0);
    for (int qd = lane; qd < G * QPR; qd += 64) {
      const int r = qd / QPR, d0 = 4 * (qd % QPR);
      float mstar = -INFINITY;
      for (int i = 0; i < n; ++i) {
        const char* ent = ring + ((f + i) % C) * EB;
        mstar = fmaxf(mstar, reinterpret_cast<const float2*>(ent + G * D * 2)[r].x);
      }
      float L = 0.f;
      f32x4 N = {0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < n; ++i) {
        const char* ent = ring + ((f + i) % C) * EB;
        const float2 ml = reinterpret_cast<const float2*>(ent + G * D * 2)[r];
        const u32x2 acc = *reinterpret_cast<const u32x2*>(ent + (r * D + d0) * 2);
        merge_fold(mstar, ml, bf16_to_acc(acc), L, N);
      }
      uint16_t* op = a.out + ((int64_t)q0 * a.num_q_heads + (kvh << a.log2_group) + r) * D + d0;
      *reinterpret_cast<u32x2*>(op) = merge_finish(N, L);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // the reads above before the entries are reused
    for (int i = lane; i < n; i += 64)
      __hip_atomic_store(&sh.gen[(f + i) % C], (f + i) / C + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  // The current task's partial into its ring entry, and the merge if it was
  // its row group's last.
  __device__ __forceinline__ void finish_task() {
    const int e = tc.j % C, want = tc.j / C;
    for (int spins = 0;; ++spins) {
      if (rfl(__hip_atomic_load(&sh.gen[e], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) == want) break;
      if (broken()) break;
      if (spins == kRgSpinLimit) {
        if (lane == 0) __hip_atomic_store(&sh.broken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    char* ent = ring + e * EB;
    const int r = lane & 15;
    if (r < G) {  // the rows of the block's one token: its G heads
      if (g4 == 0)
        reinterpret_cast<float2*>(ent + G * D * 2)[r] = make_float2(st[0].m, st[0].l());
#pragma unroll
      for (int n = 0; n < D / 16; ++n)
        *reinterpret_cast<u32x2*>(ent + (r * D + 16 * n + 4 * g4) * 2) = acc_to_bf16(st[0].acc[n]);
    }
    // (the group's size is read before the count: once the count is complete
    // another wave may merge the group and its descriptor slot be reused)
    const int n = rfl(sh.g[tc.k % kRgSlots].n);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // every lane's writes before the count
    int done = 0;
    if (lane == 0)
      done = __hip_atomic_fetch_add(&sh.g_done[tc.k % kRgSlots], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    done = rfl(done);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (done == n - 1) merge_group(tc.k);
  }

  // The next task, once the current one has at most two tiles left to compute.
  __device__ __forceinline__ void claim_next_if_due() {
    if (!have_nxt && ct + 2 >= cur.tile_end) {
      tn = claim();
      nxt = task_item(tn);
      have_nxt = true;
    }
  }

  __device__ __forceinline__ bool step(TileData<D>& Bc, TileData<D>& Bl) {
    claim_next_if_due();
    const bool in_cur = ct + 1 < cur.tile_end;
    const Item& L = in_cur ? cur : nxt;
    const int lt = in_cur ? ct + 1 : nxt.tile_begin;
    const int lend = (in_cur || nxt.valid) ? L.tile_end : lt;  // dead load past the last task
    load_tile(a, L.kvh, L.k_len, lt, lend, tile_pages(L.pt_row, L.last_entry, lt), lane, Bl);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile<D, 1>(st, Bc, curL, ct, g4, a.qk_scale_log2);
    __builtin_amdgcn_sched_barrier(0);
    if (in_cur) {
      ++ct;
      return true;
    }
    finish_task();
    if (!nxt.valid) return false;
    cur = nxt;
    tc = tn;
    have_nxt = false;
    begin_item();
    ct = cur.tile_begin;
    return true;
  }
};

template <int D>
__global__ __launch_bounds__(64 * rg_waves<D>(), 1) void attn_rowgroup_kernel(const AttnSplitArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ RgShared sh;
  __shared__ __attribute__((aligned(16))) char ring[kRgRingBytes];
  const int tid = threadIdx.x;
  for (int e = tid; e < kRgMaxEntries; e += 64 * rg_waves<D>()) sh.gen[e] = 0;
  if (tid == 0) {
    sh.lock = 0;
    sh.next_task = 0;
    sh.cur_k = -1;
    sh.cur_i = 0;
    sh.started = 0;
    sh.exhausted = 0;
    sh.static_round = 0;
    sh.broken = 0;
  }
  __syncthreads();
  const int lane = tid & 63;
  RgWave<D> w{a, sh, ring};
  w.lane = lane;
  w.g4 = lane >> 4;
  w.G = 1 << a.log2_group;
  w.C = rg_entries(D, w.G);
  w.EB = rg_entry_bytes(D, w.G);
  w.tc = w.claim();
  w.cur = w.task_item(w.tc);
  if (!w.cur.valid) return;
  w.begin_item();
  w.have_nxt = false;
  w.ct = w.cur.tile_begin;
  w.claim_next_if_due();
  TileData<D> buf0, buf1;
  load_tile(a, w.cur.kvh, w.cur.k_len, w.ct, w.cur.tile_end, tile_pages(w.cur.pt_row, w.cur.last_entry, w.ct), lane,
            buf0);
  while (w.step(buf0, buf1) && w.step(buf1, buf0)) {
  }
#endif
}

// Workgroups of the row-group kernel resident at once (per device, cached).
template <int D>
int resident_rowgroup_groups() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_rowgroup_kernel<D>, 64 * rg_waves<D>(), 0) !=
      hipSuccess)
    return 0;
  cached[dev] = max(1, cus * max(per_cu, 1));
  return cached[dev];
}

// Fewest row groups per workgroup for which the row-group mapping is taken
// (below it the split kernel's finer items balance better).
constexpr int kRgMinGroupsPerWg = 2;

// Most splits a decode row can meet: all ns, or with a window w the splits of
// w consecutive keys.
inline int rg_max_row_splits(const AttnSplitArgs& a) {
  if (a.window <= 0) return a.ns;
  const int64_t w = (int64_t)a.window + a.split - 2;
  return (int)std::min<int64_t>(a.ns, w / a.split + 1);
}

template <int D>
bool rowgroup_applies(const AttnSplitArgs& a) {
  if (a.num_tokens != a.num_seqs || a.num_seqs > kRgMaxSeqs || a.num_seqs < 1) return false;
  if (rg_max_row_splits(a) > rg_entries(D, 1 << a.log2_group)) return false;
  const int64_t groups = resident_rowgroup_groups<D>();
  if (groups <= 0) return false;
  return (int64_t)a.num_seqs * a.num_kv_heads >= groups * kRgMinGroupsPerWg;
}

// Rounds of row groups dealt statically: half of the rounds the batch makes,
// so that the smaller half of the row groups is left to the counter.  (On the
// 8B-shaped decode at batch 256, 0 to 4 static rounds of 8 measured within 1%
// of each other; all 8 static was 2% slower.)
inline int rg_static_rounds(int64_t row_groups, int64_t groups) { return (int)(row_groups / (2 * groups)); }

template <int D>
hipError_t rowgroup_launch(AttnSplitArgs a, hipStream_t stream) {
  a.qblocks = 1;
  a.spread = 0;
  const int groups = resident_rowgroup_groups<D>();
  if (groups <= 0) return hipErrorInvalidDevice;
  a.rg_static_rounds = rg_static_rounds((int64_t)a.num_seqs * a.num_kv_heads, groups);
  hipLaunchKernelGGL(attn_rowgroup_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_rowgroup_kernel<D>, dim3(groups), dim3(64 * rg_waves<D>()), 0, stream, a);
  return hipGetLastError();
}

// Workgroups of the persistent split kernel that the current device keeps
// resident at once (computed once per device, head size and item width).
template <int D, int QB>
int resident_split_groups() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_split_kernel<D, QB>, 64 * kSplitWaves, 0) !=
      hipSuccess)
    return 0;
  cached[dev] = max(1, cus * max(per_cu, 1));
  return cached[dev];
}

// Upper bound on the work items of a launch, from host-side sizes only:
// query-row blocks (at most one partial block per sequence) x KV heads x the
// splits one block can meet (all ns, or with a window the splits of w + 16
// keys).
inline int64_t item_bound(const AttnSplitArgs& a, int qb) {
  const int64_t tq = (int64_t)(kRowsPerBlock >> a.log2_group) * qb;
  // a block holds at least one token: at most num_tokens blocks (a decode batch: one per sequence)
  const int64_t blocks = std::min<int64_t>(a.num_tokens, ((int64_t)a.num_tokens + tq - 1) / tq + a.num_seqs);
  int64_t splits = a.ns;
  if (a.window > 0) splits = std::min<int64_t>(splits, (a.window + tq + a.split - 2) / a.split + 1);
  return blocks * a.num_kv_heads * splits;
}

template <int D, int QB>
hipError_t split_launch_qb(AttnSplitArgs a, hipStream_t stream) {
  a.qblocks = QB;
  const int groups = resident_split_groups<D, QB>();
  if (groups <= 0) return hipErrorInvalidDevice;
  a.spread = item_bound(a, QB) < (int64_t)groups * kSplitWaves ? 1 : 0;
  if (a.num_seqs > kLdsPlanSeqs) {
    hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_split_kernel<D, QB>), dim3(groups), dim3(64 * kSplitWaves), 0, stream, a);
  return hipGetLastError();
}

// Item width: wide items (kWideBlocks query blocks) when the batch is
// prefill-shaped — on average at least that many blocks per sequence — and
// still yields at least one wide item per resident wave (estimated with every
// row meeting all ns splits); one block otherwise.  Only the work mapping
// depends on this choice, never the arithmetic of a row.  At head_dim 256 the
// state of a second block does not fit the register file, so items stay one
// block wide.
constexpr int kWideBlocks = 4;

// Workgroups of the shared-tile kernel resident at once (per device, cached).
template <int D>
int resident_shared_groups() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_split_shared_kernel<D>, 64 * kSharedWaves, 0) !=
      hipSuccess)
    return 0;
  cached[dev] = max(1, cus * max(per_cu, 1));
  return cached[dev];
}

// Split-phase kernels by work mapping (the value is the query-row blocks per
// item); each gives every row the same bits.
constexpr int kKindOneBlock = 1;        // attn_split_kernel<D, 1>
constexpr int kKindWide = kWideBlocks;  // attn_split_kernel<D, 4>
constexpr int kKindShared = kSharedBlocks;  // attn_split_shared_kernel<D>

// The mapping for a launch: a forced one (diagnostic; 0 when it does not
// exist at this head size), else shared tiles when the batch is
// prefill-shaped (on average half an item per sequence) with an item per two
// resident workgroups; wide items when it has four blocks per sequence and an
// item per resident wave (which, given the first rule, leaves them to forced
// use); one-block items otherwise.  Item counts are host-side estimates (every row meeting all ns
// splits).
template <int D>
int split_kind(const AttnSplitArgs& a) {
  if (a.force_kind != 0) {
    if (a.force_kind == kKindOneBlock) return a.force_kind;
    if ((a.force_kind == kKindWide || a.force_kind == kKindShared) && D <= 128) return a.force_kind;
    return 0;
  }
  if constexpr (D <= 128) {
    const int64_t tq = kRowsPerBlock >> a.log2_group;  // query tokens per block
    const int64_t T = a.num_tokens, B = a.num_seqs;
    const int64_t shared_items = (T + kSharedBlocks * tq - 1) / (kSharedBlocks * tq) * a.num_kv_heads * a.ns;
    const int64_t wide_items = (T + kWideBlocks * tq - 1) / (kWideBlocks * tq) * a.num_kv_heads * a.ns;
    const int64_t wide_waves = (int64_t)resident_split_groups<D, kWideBlocks>() * kSplitWaves;
    // Shared tiles when sequences bring half an item of rows on average and
    // the items fill half a round of resident workgroups (measured: from 256
    // items of 8 blocks they beat one-block items by 7-18%, at 160 and below
    // they lose by 8-20%; at 16-24 rows per sequence they beat wide items by
    // 2-30%, and on a batch mixing decode rows with chunks by 30%, though
    // uniform 48-row chunks ran 15% faster as wide items).
    if (2 * T >= kSharedBlocks * tq * B && 2 * shared_items >= (int64_t)resident_shared_groups<D>())
      return kKindShared;
    if (T >= kWideBlocks * tq * B && wide_items >= wide_waves) return kKindWide;
  }
  return kKindOneBlock;
}

template <int D>
int item_blocks(const AttnSplitArgs& a) {
  return split_kind<D>(a);
}

template <int D>
hipError_t shared_launch(AttnSplitArgs a, hipStream_t stream) {
  a.qblocks = kSharedBlocks;
  a.spread = 0;
  int groups = resident_shared_groups<D>();
  if (groups <= 0) return hipErrorInvalidDevice;
  // Workgroup g takes items g, g + G, ...: no more workgroups than items.
  groups = (int)std::min<int64_t>(groups, std::max<int64_t>(1, item_bound(a, kSharedBlocks)));
  if (a.num_seqs > kLdsPlanSeqs) {
    hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_split_shared_kernel<D>, dim3(groups), dim3(64 * kSharedWaves), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t split_launch(const AttnSplitArgs& a, hipStream_t stream) {
  const int kind = split_kind<D>(a);
  if constexpr (D <= 128) {
    if (kind == kKindShared) return shared_launch<D>(a, stream);
    if (kind == kKindWide) return split_launch_qb<D, kWideBlocks>(a, stream);
  }
  if (kind == kKindOneBlock) return split_launch_qb<D, 1>(a, stream);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t merge_launch(const AttnMergeArgs& a, hipStream_t stream) {
  // one wave per (token, 64 threads of its rows), four waves a workgroup
  const int64_t waves = (int64_t)a.num_tokens * ((a.num_q_heads * (D / 4) + 63) / 64);
  dim3 grid((unsigned)((waves + 3) / 4));
  hipLaunchKernelGGL(attn_merge_kernel<D>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_split(int head_dim, const AttnSplitArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return split_launch<64>(a, stream);
    case 128: return split_launch<128>(a, stream);
    case 256: return split_launch<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

bool attn_rowgroup_applies(int head_dim, const AttnSplitArgs& a) {
  switch (head_dim) {
    case 64: return rowgroup_applies<64>(a);
    case 128: return rowgroup_applies<128>(a);
    case 256: return rowgroup_applies<256>(a);
    default: return false;
  }
}

hipError_t launch_attn_rowgroup(int head_dim, const AttnSplitArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return rowgroup_launch<64>(a, stream);
    case 128: return rowgroup_launch<128>(a, stream);
    case 256: return rowgroup_launch<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

int attn_item_blocks(int head_dim, const AttnSplitArgs& a) {
  switch (head_dim) {
    case 64: return item_blocks<64>(a);
    case 128: return item_blocks<128>(a);
    case 256: return item_blocks<256>(a);
    default: return 0;
  }
}

hipError_t launch_attn_merge(int head_dim, const AttnMergeArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return merge_launch<64>(a, stream);
    case 128: return merge_launch<128>(a, stream);
    case 256: return merge_launch<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bi
