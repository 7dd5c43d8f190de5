// Work distribution shared by the decode kernels: a persistent, balanced split
// of every (sequence, kv head) context over the wavefronts of one launch, and
// the in-kernel log-sum-exp merge of contexts that the split cuts.
//
// Items are (sequence, kv head) pairs, ordered sequence-major.  The context of
// an item with L tokens is cut into ceil(L / P) units of P tokens (the last one
// shorter).  With T units in all and W workers, worker w takes units
// [w*T/W, (w+1)*T/W) in that order, so every worker streams the same amount
// of cache (up to one unit) whatever the mix of context lengths.  A maximal run
// of a worker's units inside one item is a segment.  A segment that is the
// whole item is written straight to the output; otherwise the segment's
// running max m, running sum l and unnormalised output acc go to a workspace
// slot and the item's counter is incremented.  The worker that brings the
// counter to the number of segments of the item merges them:
//   M = max m_i,  out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i,
// which is the softmax over the whole context summed in another order, then
// resets the counter to zero for the next call.
//
// Each worker has two slots: slot 2w for its first segment and 2w+1 for its
// last.  Only a worker's first and last segments can be cut, so two suffice,
// and the merging worker finds every slot from the same arithmetic.
//
// Publication without cache-wide fences.  The 8 XCDs of the chip each have
// their own L2, and a device-scope fence writes back (release) or
// invalidates (acquire) a whole L2 -- thousands of those per launch cost more
// than the decode itself.  Partials are therefore written with device-scope
// atomic stores, which write through to the coherent level, and read with
// device-scope atomic loads, which read from it; the writer waits for its
// stores to complete (s_waitcnt) before it increments the counter, and the
// merger issues its loads only after the counter increment has returned.
// No other data crosses between workers.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// A launch's sequence index as (layer, sequence of the layer), and where
// that sequence's table row, context length, query, output and cache live.
__device__ __forceinline__ int layer_of(const DecodeArgs &a, int s) {
  return a.seqs_per_layer == a.num_seqs ? 0 : s / a.seqs_per_layer;  // one layer: no division
}
__device__ __forceinline__ int seq_of(const DecodeArgs &a, int s) { return s - layer_of(a, s) * a.seqs_per_layer; }
__device__ __forceinline__ int64_t q_row(const DecodeArgs &a, int s) {
  const int l = layer_of(a, s);
  return l * a.q_sl + (int64_t)(s - l * a.seqs_per_layer) * a.q_ss;
}
__device__ __forceinline__ int64_t o_row(const DecodeArgs &a, int s) {
  const int l = layer_of(a, s);
  return l * a.o_sl + (int64_t)(s - l * a.seqs_per_layer) * a.o_ss;
}
__device__ __forceinline__ int64_t k_layer(const DecodeArgs &a, int s) { return layer_of(a, s) * a.k_sl; }
__device__ __forceinline__ int64_t v_layer(const DecodeArgs &a, int s) { return layer_of(a, s) * a.v_sl; }

// The scales of item (s, kvh): qk multiplies its scores into log2 units, v
// its normalised output.  With one fp8 scale per (layer, kv head) they are
// the launch's scale * log2(e) and 1 times that head's key and value scales;
// otherwise the launch's own (per-tensor fp8 scales already folded in).
struct ItemScale {
  float qk, v;
};
__device__ __forceinline__ ItemScale item_scale(const DecodeArgs &a, int s, int kvh) {
  ItemScale r{a.qk_scale_log2, a.v_scale};
  if (a.k_head_scale != nullptr) {
    const int64_t i = (int64_t)layer_of(a, s) * a.num_kv_heads + kvh;
    r.qk *= a.k_head_scale[i];
    r.v *= a.v_head_scale[i];
  }
  return r;
}
// Only fp8 caches carry per-head scales: other kernels keep the launch's.
template <typename KVT>
__device__ __forceinline__ ItemScale seg_scale(const DecodeArgs &a, int s, int kvh) {
  if constexpr (__is_same(KVT, fp8_t)) return item_scale(a, s, kvh);
  return ItemScale{a.qk_scale_log2, a.v_scale};
}

// The split of the unit order [0, T) into Ws = min(T, W) equal ranges, range
// w worked by worker w (never more ranges than units, so none is empty).
struct Split {
  int64_t T, Ws;
  // first unit of range p, and the range that holds unit x
  __device__ __forceinline__ int64_t begin(int64_t p) const { return p * T / Ws; }
  __device__ __forceinline__ int64_t owner(int64_t x) const { return ((x + 1) * Ws - 1) / T; }
};

__device__ __forceinline__ Split make_split(int64_t T, int64_t W) {
  Split sp;
  sp.T = T;
  sp.Ws = T < W ? T : W;
  return sp;
}

// A window of 64 consecutive sequences: units per sequence and their prefix sums.
struct SeqWindow {
  int s0;        // first sequence of the window
  int L;         // this lane's sequence: clamped context length (0 past the last sequence)
  int n;         // this lane's sequence: number of units
  int incl;      // inclusive prefix of n inside the window
  int total;     // units of the whole window (uniform)
};

__device__ __forceinline__ SeqWindow load_window(const DecodeArgs &a, int s0, int lane) {
  SeqWindow win;
  win.s0 = s0;
  const int s = s0 + lane;
  win.L = s < a.num_seqs ? clamp_ctx(a.context_lens[seq_of(a, s)], a.max_ctx) : 0;
  win.n = (win.L + a.part_tokens - 1) / a.part_tokens;
  win.incl = wave_incl_scan(win.n, lane);
  win.total = uniform(__shfl(win.incl, 63));
  return win;
}

// The first kWin windows (sequences 0 .. 64 kWin - 1), loaded together when a
// worker starts; windows past them are loaded one by one when needed.
constexpr int kWin = 4;
struct Windows {
  SeqWindow w[kWin];
  int nw;  // windows held: min(kWin, ceil(num_seqs / 64))
};

__device__ __forceinline__ void load_windows(const DecodeArgs &a, int lane, Windows &ws) {
  int L[kWin];
  // all loads in flight together: every lane loads (lanes past the last
  // sequence read the last one's length again), and the lengths are chosen
  // afterwards -- a load under a per-lane condition would be awaited before
  // the next one is issued
#pragma unroll
  for (int i = 0; i < kWin; ++i) L[i] = a.context_lens[seq_of(a, min(64 * i + lane, a.num_seqs - 1))];
#pragma unroll
  for (int i = 0; i < kWin; ++i) L[i] = 64 * i + lane < a.num_seqs ? clamp_ctx(L[i], a.max_ctx) : 0;
  ws.nw = 0;
#pragma unroll
  for (int i = 0; i < kWin; ++i) {
    SeqWindow &win = ws.w[i];
    win.s0 = 64 * i;
    win.L = L[i];
    win.n = (win.L + a.part_tokens - 1) / a.part_tokens;
    win.incl = wave_incl_scan(win.n, lane);
    win.total = uniform(__shfl(win.incl, 63));
    if (64 * i < a.num_seqs) ws.nw = i + 1;
  }
}

// Partials cross between wavefronts of different XCDs.  They are written and
// read through buffer descriptors over the two workspace regions with the
// device-coherent cache policy (sc1, the policy of device-scope atomic
// stores and loads: writes go through to the coherent level past every XCD's
// own L2, reads come from it), 16 bytes per access, so a wave's accesses
// cover whole lines; an access outside a region is dropped by the
// descriptor's bound.
constexpr int kCoherent = 16;  // cache-policy operand: sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t region(float *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void store_shared4(const DecodeArgs &a, int64_t elem, const float *x) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(uint32_t, x[i]);
  __builtin_amdgcn_raw_buffer_store_b128(v, region(a.part_acc, a.acc_bytes), (uint32_t)(elem * 4), 0, kCoherent);
}
__device__ __forceinline__ u32x4 load_shared4(const DecodeArgs &a, int64_t elem) {
  return __builtin_amdgcn_raw_buffer_load_b128(region(a.part_acc, a.acc_bytes), (uint32_t)(elem * 4), 0, kCoherent);
}
__device__ __forceinline__ void store_shared_ml(const DecodeArgs &a, int64_t elem, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), region(a.part_ml, a.ml_bytes),
                                        (uint32_t)(elem * 4), 0, kCoherent);
}
__device__ __forceinline__ float load_shared_ml(const DecodeArgs &a, int64_t elem) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(region(a.part_ml, a.ml_bytes),
                                                                        (uint32_t)(elem * 4), 0, kCoherent));
}

// Where the partial of a slot lives: G * D unnormalised outputs (head-major)
// and G (max, sum) pairs, in elements of the two regions.
template <int G, int D>
__device__ __forceinline__ int64_t slot_acc(int64_t slot) { return slot * (int64_t)(G * D); }
template <int G>
__device__ __forceinline__ int64_t slot_ml(int64_t slot) { return slot * (int64_t)(G * 2); }

template <typename QT>
__device__ __forceinline__ void store_elem(const DecodeArgs &a, int64_t idx, float x) {
  if (a.out_f32)
    reinterpret_cast<float *>(a.out)[idx] = x;
  else
    Elem<QT>::store(a.out, idx, x);
}

// Merge the segments of item (s, kvh) whose units start at a0 (n units): the
// caller is the last of its workers to finish.  The partials are read in
// batches of up to PB, all loads of a batch in flight together, and folded
// into a running (M, L, O) per output element, so a merge costs about one
// memory round trip per batch.  Lane l owns the 16-byte vectors l + 64 k of
// the [G][D] block (4 outputs of one head each); the (max, sum) pairs of a
// partial are read by lanes 0 .. 2G-1 and passed to the lanes that need them.
template <typename QT, int G, int D>
__device__ void merge_item(const DecodeArgs &a, int s, int kvh, int64_t a0, int64_t n, const Split &sp, int lane) {
  constexpr int NV = G * D / 4;        // vectors of a partial's outputs
  constexpr int VPL = (NV + 63) / 64;  // per lane
  constexpr int PB0 = 96 / (4 * VPL + 1);
  constexpr int PB = PB0 < 1 ? 1 : (PB0 > 8 ? 8 : PB0);  // partials per batch: up to ~96 registers of loads
  static_assert(D % 4 == 0 && 2 * G <= 64, "a vector stays inside one head; a lane per (max, sum) value");
  const int64_t w0 = sp.owner(a0), w1 = sp.owner(a0 + n - 1);
  const bool first_is_last = sp.begin(w0) < a0;  // range w0 began in an earlier item
  const int cnt = (int)(w1 - w0 + 1);
  float M[VPL], L[VPL], O[VPL][4];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    M[k] = -INFINITY;
    L[k] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) O[k][i] = 0.0f;
  }
  for (int i0 = 0; i0 < cnt; i0 += PB) {
    float bml[PB];
    u32x4 bacc[PB][VPL];
#pragma unroll
    for (int b = 0; b < PB; ++b) {
      if (i0 + b >= cnt) break;
      const int64_t wi = w0 + i0 + b;
      const int64_t slot = (i0 + b == 0 && first_is_last) ? 2 * wi + 1 : 2 * wi;
      bml[b] = lane < 2 * G ? load_shared_ml(a, slot_ml<G>(slot) + lane) : 0.0f;
#pragma unroll
      for (int k = 0; k < VPL; ++k)
        if (lane + 64 * k < NV) bacc[b][k] = load_shared4(a, slot_acc<G, D>(slot) + 4 * (lane + 64 * k));
    }
#pragma unroll
    for (int b = 0; b < PB; ++b) {
      if (i0 + b >= cnt) break;
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        int g = (4 * (lane + 64 * k)) / D;
        g = g < G ? g : G - 1;
        const float mi = __shfl(bml[b], 2 * g), li = __shfl(bml[b], 2 * g + 1);
        if (lane + 64 * k < NV) {
          const float mn = fmaxf(M[k], mi);
          const float f0 = fast_exp2(M[k] - mn), f1 = fast_exp2(mi - mn);
          L[k] = L[k] * f0 + li * f1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t x = bacc[b][k][i];
            O[k][i] = O[k][i] * f0 + __builtin_bit_cast(float, x) * f1;
          }
          M[k] = mn;
        }
      }
    }
  }
  const float vsc = item_scale(a, s, kvh).v;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    if (lane + 64 * k >= NV) continue;
    const int e = 4 * (lane + 64 * k);
    const int head = kvh * G + e / D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      store_elem<QT>(a, o_row(a, s) + (int64_t)head * a.o_sh + e % D + i, O[k][i] / L[k] * vsc);
  }
}

// Count a segment's partial (already stored by the caller to its slot, and
// those stores complete) and, if it is the item's last, merge.  All lanes call.
template <typename QT, int G, int D>
__device__ __forceinline__ void publish_partial(const DecodeArgs &a, int s, int kvh, int64_t a0, int64_t n,
                                                const Split &sp, int lane) {
  const int64_t w0 = sp.owner(a0), w1 = sp.owner(a0 + n - 1);
  const int cnt = (int)(w1 - w0 + 1);
  int32_t *ctr = a.counters + (int64_t)s * a.num_kv_heads + kvh;
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = uniform(__shfl(old, 0));
  if (old == cnt - 1) {
    // every other segment's count, hence its stores, came before ours
    merge_item<QT, G, D>(a, s, kvh, a0, n, sp, lane);
    if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait for the partial's write-through stores, then count it (the signal
// fences keep the compiler from moving memory operations across the wait).
template <typename QT, int G, int D>
__device__ __forceinline__ void finish_partial(const DecodeArgs &a, int s, int kvh, int64_t a0, int64_t n,
                                               const Split &sp, int lane) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  publish_partial<QT, G, D>(a, s, kvh, a0, n, sp, lane);
}

// The cache write of a fused step (pa_decode_append): every sequence's new
// K and V rows, split into row pieces of one kv head (head_dim elements,
// LPP lanes of 16 bytes each), piece p handled by lane group p % PPI of
// worker (p / PPI) % W.  A worker loads its first pieces with the context
// lengths it loads at its start (so they add no wait of their own) and
// stores them when it has finished its decode work, so no store is pending
// while its load pipeline runs; pieces past the first W * PPI (large batches)
// are copied then too, one load and store each.  Slots < 0 or past the pool
// are skipped, and so are sequences with an empty context.  No worker reads a
// slot being written here: the decode takes the new token's rows from k_new /
// v_new.
template <int D, int EB>
struct AppendRows {
  static constexpr int LPP = D * EB / 16;  // lanes per piece
  static constexpr int PPI = 64 / LPP;     // pieces per wave-wide instruction
  static_assert(LPP >= 1 && LPP <= 64 && 64 % LPP == 0, "a piece is a whole number of lanes");
  u32x4 v;
  int64_t p;
  uint32_t slot_lo, slot_hi;  // the slot's two 32-bit halves (an int32 slot: its value twice)
  int ctx;

  // Issue the loads of piece p (this lane's 16 bytes, the slot, the length);
  // nothing here waits for them.  Every lane loads -- a piece past the last
  // reads the last one's again, and store() skips it -- and through pointers
  // the compiler knows to be global: a load under a per-lane condition was
  // awaited at once, and a flat one made the next wait for a scalar load
  // wait for it too, each a memory round trip ahead of the decode work.
  __device__ __forceinline__ void load(const DecodeArgs &a, int64_t piece, int lane) {
    p = piece;
    const int64_t pieces = 2 * (int64_t)a.num_seqs * a.num_kv_heads;
    const int64_t q = p < pieces ? p : pieces - 1;
    const int kvh = (int)(q % a.num_kv_heads);
    const bool is_v = (q / a.num_kv_heads) & 1;
    const int64_t n = q / (2 * (int64_t)a.num_kv_heads);
    const int64_t c = (int64_t)(lane % LPP) * (16 / EB);  // this lane's element of the row
    // both candidate addresses as values (a choice between fields of the
    // kernel's argument block would place that block in private memory), the
    // load through a global-memory pointer made from the chosen one
    typedef const __attribute__((address_space(1))) u32x4 global_u32x4;
    const uintptr_t src_k = (uintptr_t)a.k_new + (uintptr_t)((n * a.kn_ss + kvh * a.kn_sh + c) * EB);
    const uintptr_t src_v = (uintptr_t)a.v_new + (uintptr_t)((n * a.vn_ss + kvh * a.vn_sh + c) * EB);
    v = *reinterpret_cast<global_u32x4 *>(is_v ? src_v : src_k);
    const char *sp = static_cast<const char *>(a.slot_mapping) + n * (a.slot_i64 ? 8 : 4);
    slot_lo = *reinterpret_cast<const uint32_t *>(sp);
    slot_hi = *reinterpret_cast<const uint32_t *>(sp + (a.slot_i64 ? 4 : 0));
    ctx = a.context_lens[n];
  }
  // Store the piece to its slot (after the loads have arrived).
  __device__ __forceinline__ void store(const DecodeArgs &a, int lane) const {
    const int64_t slot = a.slot_i64 ? (int64_t)(((uint64_t)slot_hi << 32) | slot_lo) : (int64_t)(int32_t)slot_lo;
    if (p >= 2 * (int64_t)a.num_seqs * a.num_kv_heads || slot < 0 || slot >= a.num_slots || ctx <= 0) return;
    const int kvh = (int)(p % a.num_kv_heads);
    const bool is_v = (p / a.num_kv_heads) & 1;
    const int64_t c = (int64_t)(lane % LPP) * (16 / EB);
    const int64_t blk = slot / a.block_size, off = slot % a.block_size;
    const uintptr_t dst_k = (uintptr_t)a.k_cache + (uintptr_t)((blk * a.k_sb + off * a.k_st + kvh * a.k_sh + c) * EB);
    const uintptr_t dst_v = (uintptr_t)a.v_cache + (uintptr_t)((blk * a.v_sb + off * a.v_st + kvh * a.v_sh + c) * EB);
    st16(reinterpret_cast<void *>(is_v ? dst_v : dst_k), v);
  }
};

// A fused step writes sequence s's new token only to a slot inside the pool;
// only then does the decode take that token's rows from the new rows (a
// skipped slot leaves the cache as it stands, and the decode reads it).
__device__ __forceinline__ bool append_writes(const DecodeArgs &a, int s) {
  typedef const __attribute__((address_space(4))) int64_t c64;
  typedef const __attribute__((address_space(4))) int32_t c32;
  const int64_t slot = a.slot_i64 ? ((c64 *)(uintptr_t)a.slot_mapping)[s] : (int64_t)((c32 *)(uintptr_t)a.slot_mapping)[s];
  return slot >= 0 && slot < a.num_slots;
}

// Zero the output rows of sequences with an empty context (sequence s is
// handled by worker s mod W).
template <typename QT>
__device__ __forceinline__ void zero_empty_sequences(const DecodeArgs &a, const SeqWindow &win, int w, int W,
                                                     int lane) {
  const int s = win.s0 + lane;
  const bool mine = s < a.num_seqs && win.n == 0 && (s % W) == w;
  uint64_t mask = __ballot(mine);
  while (mask) {
    const int l = __builtin_ctzll(mask);
    mask &= mask - 1;
    const int sz = win.s0 + l;
    for (int e = lane; e < a.num_heads * a.head_dim; e += 64)
      store_elem<QT>(a, o_row(a, sz) + (int64_t)(e / a.head_dim) * a.o_sh + e % a.head_dim, 0.0f);
  }
}

// Where unit x sits: its sequence, the first unit of that sequence's kv head
// 0, the sequence's units per kv head and its context length (all uniform).
struct UnitPos {
  int s;
  int n;
  int L;
  int64_t item0;
};

// Unit x of window `win`, whose first unit is base + (units of its earlier
// sequences); false if x is not in it.
__device__ __forceinline__ bool locate_in(const DecodeArgs &a, const SeqWindow &win, int64_t base, int64_t x,
                                          UnitPos &p) {
  const int64_t lo = base + (int64_t)(win.incl - win.n) * a.num_kv_heads;
  const int64_t hi = base + (int64_t)win.incl * a.num_kv_heads;
  const uint64_t hit = __ballot(win.n > 0 && lo <= x && x < hi);
  if (hit == 0) return false;
  const int ls = __builtin_ctzll(hit);
  p.s = win.s0 + ls;
  p.n = uniform(__shfl(win.n, ls));
  p.L = uniform(__shfl(win.L, ls));
  p.item0 = base + (int64_t)uniform(__shfl(win.incl - win.n, ls)) * a.num_kv_heads;
  return true;
}

// Find unit x (x < T): the held windows first, then the windows after them.
// Returns false only if the context lengths changed under the launch.
__device__ __forceinline__ bool locate(const DecodeArgs &a, const Windows &ws, int64_t x, int lane, UnitPos &p) {
  int64_t base = 0;  // units (all kv heads) of the sequences before the window
#pragma unroll
  for (int i = 0; i < kWin; ++i) {
    if (i < ws.nw) {
      const int64_t units = (int64_t)ws.w[i].total * a.num_kv_heads;
      if (x < base + units) return locate_in(a, ws.w[i], base, x, p);
      base += units;
    }
  }
  for (int s0 = 64 * ws.nw; s0 < a.num_seqs; s0 += 64) {
    const SeqWindow win = load_window(a, s0, lane);
    const int64_t units = (int64_t)win.total * a.num_kv_heads;
    if (x < base + units) return locate_in(a, win, base, x, p);
    base += units;
  }
  return false;
}

// One segment of a worker's range: units [u_lo, u_hi) of item (s, kvh), as
// tokens [t_lo, t_hi), plus what finishing it needs.
struct SegInfo {
  int s, kvh;
  int t_lo, t_hi;
  int u_lo, u_hi, n;  // units of the segment; units per kv head of the sequence
  int64_t a0;         // first unit of the item
  bool first;         // the first segment of the range (slot 2w) rather than a later one (2w+1)
};

// Yields a worker's segments in the order: the range's last segment, its
// first, then the whole items between them.  A context cut between workers w
// and w+1 is then the first or second thing both of them do, so its merge
// happens early in the launch instead of in its tail.
struct Walker {
  const DecodeArgs *ap;
  int64_t b, e, a0_b, end_b, a0_e;
  UnitPos pb, pe, p;
  int kvh_b, kvh_e, kvh;
  int stage;  // 0: last segment next, 1: first segment next, 2: whole items, 3: done
  int64_t x;  // next unit of stage 2

  __device__ explicit Walker(const DecodeArgs &args) : ap(&args) {}

  // false if there is nothing to do (or context_lens changed under the launch)
  __device__ bool init(const Windows &first, int64_t b_, int64_t e_, int lane) {
    const DecodeArgs &a = *ap;
    b = b_;
    e = e_;
    if (!locate(a, first, b, lane, pb)) return false;
    kvh_b = (int)((b - pb.item0) / pb.n);
    a0_b = pb.item0 + (int64_t)kvh_b * pb.n;
    end_b = a0_b + pb.n;
    stage = 1;
    if (e > end_b) {
      if (!locate(a, first, e - 1, lane, pe)) return false;
      kvh_e = (int)((e - 1 - pe.item0) / pe.n);
      a0_e = pe.item0 + (int64_t)kvh_e * pe.n;
      stage = 0;
    }
    return true;
  }

  __device__ void fill(SegInfo &g, const UnitPos &q, int kv, int u_lo, int u_hi, bool is_first) const {
    const DecodeArgs &a = *ap;
    g.s = q.s;
    g.kvh = kv;
    g.u_lo = u_lo;
    g.u_hi = u_hi;
    g.n = q.n;
    g.a0 = q.item0 + (int64_t)kv * q.n;
    g.t_lo = u_lo * a.part_tokens;
    g.t_hi = (int)((int64_t)u_hi * a.part_tokens < q.L ? (int64_t)u_hi * a.part_tokens : q.L);
    g.first = is_first;
  }

  __device__ bool next(SegInfo &g) {
    const DecodeArgs &a = *ap;
    if (stage == 0) {
      fill(g, pe, kvh_e, 0, (int)(e - a0_e), false);
      stage = 1;
      return true;
    }
    if (stage == 1) {
      fill(g, pb, kvh_b, (int)(b - a0_b), (int)((e < end_b ? e : end_b) - a0_b), true);
      stage = e > end_b ? 2 : 3;
      p = pb;
      kvh = kvh_b;
      x = end_b;
      return true;
    }
    if (stage == 3 || x >= a0_e) {
      stage = 3;
      return false;
    }
    // the item after (p, kvh): the next kv head, else the next sequence with a non-empty context
    if (++kvh == a.num_kv_heads) {
      kvh = 0;
      p.item0 += (int64_t)p.n * a.num_kv_heads;
      do {
        if (++p.s >= a.num_seqs) {  // only if context_lens changed under the launch
          stage = 3;
          return false;
        }
        p.L = clamp_ctx(uniform(a.context_lens[seq_of(a, p.s)]), a.max_ctx);
        p.n = (p.L + a.part_tokens - 1) / a.part_tokens;
      } while (p.n == 0);
    }
    fill(g, p, kvh, 0, p.n, false);
    x += p.n;
    return true;
  }
};

// Drive one worker through its range.  Seg must provide
//   void begin(const SegInfo &g, const Walker &from)        -- issue the loads of g's first chunk(s);
//       `from` yields the worker's segments from g on, for loads that run
//       more than one segment ahead
//   void run(const SegInfo &g, const SegInfo &nx, bool has) -- attend over g's tokens (its first chunk
//       already in flight); while on g's last chunk, issue nx's first chunk if `has`
//   void write_out(int s, int kvh)                          -- normalised output of a whole item
//   void write_partial(int64_t slot)                        -- partial (m, l, acc) to a slot
//   void publish(const SegInfo &g, const Split &sp)         -- count g's partial (finish_partial, now or
//       once its stores are known complete)
//   void end()                                              -- after the last segment (publishes what is left)
// All lanes of the wave call every function; all control flow is uniform.
// The load pipeline thus runs on from one segment into the next.
// Total units T of the launch (all kv heads); zeroes the outputs of empty
// sequences on the way.
template <typename QT>
__device__ int64_t count_units(const DecodeArgs &a, int w, int W, int lane, Windows &first) {
  int64_t T = 0;
  load_windows(a, lane, first);
#pragma unroll
  for (int i = 0; i < kWin; ++i) {
    if (i < first.nw) {
      zero_empty_sequences<QT>(a, first.w[i], w, W, lane);
      T += (int64_t)first.w[i].total;
    }
  }
  for (int s0 = 64 * first.nw; s0 < a.num_seqs; s0 += 64) {
    const SeqWindow win = load_window(a, s0, lane);
    zero_empty_sequences<QT>(a, win, w, W, lane);
    T += (int64_t)win.total;
  }
  return T * a.num_kv_heads;
}

// A fused step's copy of the new rows around a worker's decode work: its
// first pieces loaded before the work starts, stored (and the rest copied)
// after it ends.
template <int D, int EB>
struct AppendCopy {
  typedef AppendRows<D, EB> Rows;
  Rows rows;
  __device__ __forceinline__ void begin(const DecodeArgs &a, int w, int lane) {
    rows.load(a, (int64_t)w * Rows::PPI + lane / Rows::LPP, lane);
  }
  __device__ __forceinline__ void end(const DecodeArgs &a, int w, int W, int lane) {
    rows.store(a, lane);
    const int64_t pieces = 2 * (int64_t)a.num_seqs * a.num_kv_heads;
    for (int64_t p0 = ((int64_t)W + w) * Rows::PPI; p0 < pieces; p0 += (int64_t)W * Rows::PPI) {
      rows.load(a, p0 + lane / Rows::LPP, lane);
      rows.store(a, lane);
    }
  }
};

template <typename QT, int G, int D, class Seg, int APPEND_EB = 0>
__device__ __forceinline__ void run_worker(const DecodeArgs &a, int w, int W, int lane, Seg &seg) {
  if constexpr (APPEND_EB > 0) {
    AppendCopy<D, APPEND_EB> copy;
    copy.begin(a, w, lane);
    run_worker<QT, G, D, Seg, 0>(a, w, W, lane, seg);
    copy.end(a, w, W, lane);
    return;
  }
  Windows first;
  const Split sp = make_split(count_units<QT>(a, w, W, lane, first), W);
  if (w >= sp.Ws) return;

  Walker walk(a);
  if (!walk.init(first, sp.begin(w), sp.begin(w + 1), lane)) return;
  const Walker from = walk;
  SegInfo cur, nx;
  if (!walk.next(cur)) return;
  seg.begin(cur, from);
  bool has = walk.next(nx);
  while (true) {
    seg.run(cur, nx, has);
    if (cur.u_lo == 0 && cur.u_hi == cur.n) {
      seg.write_out(cur.s, cur.kvh);
    } else {
      seg.write_partial(cur.first ? 2 * (int64_t)w : 2 * (int64_t)w + 1);
      seg.publish(cur, sp);
    }
    if (!has) break;
    cur = nx;
    has = walk.next(nx);
  }
  seg.end();
}

}  // namespace pa
