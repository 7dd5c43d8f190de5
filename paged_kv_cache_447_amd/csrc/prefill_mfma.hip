// Paged prefill on the matrix cores: several query tokens per sequence (a
// prompt chunk, or the draft tokens of a speculative step), each attending
// causally to the cached context up to its own position.
//
// The query rows of a sequence are its newest tokens; their K/V rows are
// already in the cache (written by the cache-write scatter), so every score
// reads K and V through the block table exactly as decode does: logical block
// t / block_size to physical block, offset t % block_size (page
// "vLLM框架中的KV cache优化与PagedAttention机制详解", section 5.1; address rule of
// page "Paged KVCache：大模型推理显存管理优化方案", section 2.3).  The query tensor
// holds one row per token of the step, as in the kernel interface of page
// "vLLM推理引擎架构：PagedAttention机制与高吞吐推理" (section 2.3), and a prompt
// takes ceil(prompt_len / block_size) blocks (section 2.2 of the same page).
//
// Work: the columns of a (sequence, kv head) pair are its (query row, query
// head) pairs, row-major with the G heads of the group; each workgroup of 4
// wavefronts computes a tile of 4 x 16 NC columns, each wavefront 16 NC of
// them as NC MfmaCore column sets (mfma_core.h).  A column's scores are masked
// past its own position, so one chunk pass serves rows with different limits.
// The workgroup streams the K and V rows of positions 0 .. (its last row's
// position) in 32-token chunks through an LDS ring of R slots (80 KB, so that
// two workgroups share a CU): each wavefront loads a quarter of every chunk
// straight from HBM into LDS, and one barrier per chunk both publishes a chunk
// to all four wavefronts and frees the slot that the next loads go into, so
// R - 1 chunks are in flight during each chunk's arithmetic.  Every wavefront reads the K operands and transposed V
// operands of the chunk from LDS and multiplies them into all NC of its
// column sets.
#include "mfma_core.h"
#include "pa_internal.h"

namespace pa {

namespace {

using namespace mfma;

constexpr int kWaves = 4;            // wavefronts per workgroup, sharing one K/V stream
constexpr int kLdsPerWG = 80 * 1024;  // two workgroups per CU share its 160 KB of LDS

typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ lds_void *lds_addr(char *p) { return (lds_void *)p; }

// A workgroup barrier without the memory fence of __syncthreads(), whose
// wait for every outstanding load would drain the ring; the chunk loads are
// awaited explicitly before it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Query rows [lo, hi) of sequence i (clamped into [0, num_rows]).
__device__ __forceinline__ void seq_rows(const PrefillArgs &a, int i, int &lo, int &hi) {
  lo = clampi(a.query_start_loc[i], 0, a.num_rows);
  hi = clampi(a.query_start_loc[i + 1], lo, a.num_rows);
}

__device__ __forceinline__ int seq_tiles(const PrefillArgs &a, int i) {
  int lo, hi;
  seq_rows(a, i, lo, hi);
  return (int)(((int64_t)(hi - lo) * a.group + a.tile_cols - 1) / a.tile_cols);
}

// The order of the tiles.  Every sequence has ceil(rows * G / tile_cols)
// tiles, its last tile (whose rows see the most positions) first.  Batches of
// up to kRanked sequences take their sequences longest context first (ties in
// sequence order), so that the longest work starts first: the lengths are
// loaded once, in one round trip, and ranked in registers.  Larger batches
// keep their own order and are scanned for each tile.  All results are
// wave-uniform.
struct TileOrder {
  static constexpr int kWin = 4;
  static constexpr int kRanked = 64 * kWin;
  bool ranked;
  int total;                      // tiles of all sequences (ranked batches)
  int tiles[kWin], before[kWin];  // per lane: its sequence's tiles, and those of the sequences ranked before it

  __device__ __forceinline__ void init(const PrefillArgs &a, int lane) {
    ranked = a.num_seqs <= kRanked;
    total = 0;
    if (!ranked) return;
    int L[kWin];
#pragma unroll
    for (int w = 0; w < kWin; ++w) {
      const int i = 64 * w + lane;
      tiles[w] = 0;
      L[w] = -1;
      before[w] = 0;
      if (i < a.num_seqs) {
        tiles[w] = seq_tiles(a, i);
        L[w] = clamp_ctx(a.context_lens[i], a.max_ctx);
      }
    }
    rank_against<0>(a, lane, L);
    rank_against<1>(a, lane, L);
    rank_against<2>(a, lane, L);
    rank_against<3>(a, lane, L);
    static_assert(kWin == 4, "one rank_against per window");
  }

  // Count, for every lane's sequence, the tiles of window W2's sequences that
  // rank before it (a template per window keeps every array index static).
  template <int W2>
  __device__ __forceinline__ void rank_against(const PrefillArgs &a, int lane, const int *L) {
    if (64 * W2 >= a.num_seqs) return;
    const int n = min(64, a.num_seqs - 64 * W2);
    const int Lw = L[W2], tw = tiles[W2];
    for (int k = 0; k < n; ++k) {
      const int Lk = __builtin_amdgcn_readlane(Lw, k), tk = __builtin_amdgcn_readlane(tw, k);
      total += tk;
#pragma unroll
      for (int w = 0; w < kWin; ++w)
        if (64 * w < a.num_seqs) before[w] += (Lk > L[w] || (Lk == L[w] && 64 * W2 + k < 64 * w + lane)) ? tk : 0;
    }
  }

  // Tile number t among window W's sequences (ranked batches)
  template <int W>
  __device__ __forceinline__ bool find_in(int t, int &seq, int &tile) const {
    const uint64_t hit = __ballot(tiles[W] > 0 && before[W] <= t && t < before[W] + tiles[W]);
    if (!hit) return false;
    const int k = __builtin_ctzll(hit);
    seq = 64 * W + k;
    tile = __builtin_amdgcn_readlane(before[W] + tiles[W], k) - 1 - t;
    return true;
  }

  // The sequence and tile of tile number t; false past the last tile.
  __device__ __forceinline__ bool find(const PrefillArgs &a, int t, int lane, int &seq, int &tile) const {
    if (ranked)
      return find_in<0>(t, seq, tile) || find_in<1>(t, seq, tile) || find_in<2>(t, seq, tile) ||
             find_in<3>(t, seq, tile);
    int carry = 0;
    for (int base = 0; base < a.num_seqs; base += 64) {
      const int i = base + lane;
      const int nt = i < a.num_seqs ? seq_tiles(a, i) : 0;
      const int incl = wave_incl_scan(nt, lane);
      const int tot = uniform(__shfl(incl, 63));
      if (t < carry + tot) {
        const int k = uniform(__builtin_ctzll(__ballot(carry + incl > t)));
        seq = base + k;
        tile = uniform(__shfl(incl, k)) - 1 - (t - carry);
        return true;
      }
      carry += tot;
    }
    return false;
  }
};

// KSP (key split): for tiles of few columns (verification-sized steps), the
// four wavefronts all compute the tile's 16 NC columns, each over every fourth
// chunk, which it loads alone into a private two-slot ring; the four partial
// softmax states are merged through LDS at the end.  Otherwise the four
// wavefronts compute different columns over every chunk of one shared stream.
// BSC: fp8 caches with one scale per (block, kv head) (a variant of its own,
// so that the other launches carry none of its work)
template <typename MT, typename KVT, int D, int BS, int NC, bool KSP, bool BSC = false>
struct PrefillTile {
  using Slot = RowSlot<D>;
  static constexpr bool kFp8 = __is_same(KVT, fp8_t);
  static constexpr int EB = kFp8 ? 1 : 2;             // bytes per cache element
  static constexpr int PPR = D * EB / 16;             // 16-byte pieces per cache row
  using Core = MfmaCore<MT, D>;
  static constexpr int KS = D / 32;
  static constexpr int NT = D / 16;
  static constexpr int RB = Slot::RB;
  static constexpr int HB = Slot::HB;                 // bytes of the K (or V) rows of a chunk
  static constexpr int PER = Slot::NLD / kWaves;      // DMA instructions per wavefront per K (or V) chunk
  static constexpr int CB = 2 * HB;                   // bytes of a ring slot: K rows, then V rows
  static constexpr int R = kLdsPerWG / CB < 8 ? kLdsPerWG / CB : 8;  // ring slots (shared stream)
  // key split: two private slots per wavefront, reused for the partials' merge
  // merge buffer: a column's D outputs padded to PD floats, so that the 16
  // columns of one 16-byte access fall on 16 different bank groups
  static constexpr int PD = D + 4;
  static constexpr int kMergeBytes = kWaves * NC * 16 * (PD + 2) * 4;
  static constexpr int kLdsBytes = KSP ? kWaves * 2 * CB : R * CB;
  static_assert(!KSP || kMergeBytes <= kLdsBytes, "the partials fit the ring");
  static_assert(!KSP || 3 * Slot::NLD < 64, "wait counter range");
  static constexpr int LOG2BS = BS == 16 ? 4 : 5;
  static_assert(Slot::NLD % kWaves == 0, "every wavefront loads the same share of a chunk");
  static_assert(Slot::RPI * PER == 8, "a wavefront's share is 8 rows inside one 16-token tile");
  static_assert(R >= 3 && 2 * (R - 2) * PER < 64, "ring depth within the wait counter's range");

  const PrefillArgs &a;
  char *const ring;
  const int lane, wave, c16, jq;

  // the workgroup's tile
  int s, kvh, q0, pos0, c_hi, last_max;
  float qk_sc, v_sc;  // its score scale (log2 units) and output scale: the launch's, or its fp8 kv head's
  const float *ksb, *vsb;  // fp8 per-block scales of its kv head (stride num_kv_heads per block), or null
  const_i32 *bt;
  const char *kbase, *vbase;
  // this wavefront's columns
  int wlast;          // last position any of them sees (-1: no columns)
  int last[NC];       // per lane: the position its column sees up to
  int row[NC], head[NC];
  bool valid[NC];
  u32x4 qop[NC][KS];
  Core core[NC];
  int koff[KS], voff[NT];

  __device__ PrefillTile(const PrefillArgs &args, char *lds, int ln, int wv)
      : a(args), ring(lds), lane(ln), wave(wv), c16(ln & 15), jq(ln >> 4) {
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) koff[kb] = Slot::k_off(c16, jq, kb);
#pragma unroll
    for (int n = 0; n < NT; ++n) voff[n] = Slot::v_off(c16, jq, n);
  }

  // Set up tile `tile` of sequence `seq` for kv head `kh`; false if none of
  // its rows sees a position (then its outputs are written as zeros).
  __device__ bool setup(int seq, int tile, int kh) {
    s = seq;
    kvh = kh;
    qk_sc = a.qk_scale_log2;
    v_sc = a.v_scale;
    ksb = vsb = nullptr;
    if constexpr (kFp8) {
      if (a.k_head_scale != nullptr) {
        qk_sc *= a.k_head_scale[kvh];
        v_sc *= a.v_head_scale[kvh];
      }
      if (BSC) {
        ksb = a.k_block_scale + kvh;
        vsb = a.v_block_scale + kvh;
      }
    }
    int q1;
    seq_rows(a, s, q0, q1);
    const int nq = q1 - q0;
    const int L = clamp_ctx(a.context_lens[s], a.max_ctx);
    pos0 = L - nq;  // position of the sequence's first query row
    const int c_lo = tile * a.tile_cols;
    c_hi = min(c_lo + a.tile_cols, nq * a.group);
    last_max = pos0 + (c_hi - 1) / a.group;
    bt = as_const(a.block_tables) + (int64_t)s * a.bt_ss;
    kbase = reinterpret_cast<const char *>(a.k_cache) + (int64_t)kvh * a.k_sh * EB;
    vbase = reinterpret_cast<const char *>(a.v_cache) + (int64_t)kvh * a.v_sh * EB;
    const int w_lo = KSP ? c_lo : c_lo + 16 * NC * wave;
    wlast = w_lo < c_hi ? pos0 + (min(w_lo + 16 * NC, c_hi) - 1) / a.group : -1;
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      const int col = w_lo + 16 * ct + c16;
      valid[ct] = col < c_hi;
      const int r = valid[ct] ? col / a.group : 0;
      row[ct] = q0 + r;
      head[ct] = kvh * a.group + (valid[ct] ? col - r * a.group : 0);
      // padding columns (never written) run with the tile's limit
      last[ct] = valid[ct] ? pos0 + r : last_max;
    }
    return last_max >= 0;
  }

  // q^T operands: lane (c16, jq) of set ct holds q[row][head][32 kb + 8 jq ..]
  // (a padding column holds the tile's first row: finite, never written)
  __device__ __forceinline__ void load_q() {
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      const uint16_t *qr =
          reinterpret_cast<const uint16_t *>(a.q) + (int64_t)row[ct] * a.q_sn + (int64_t)head[ct] * a.q_sh;
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) qop[ct][kb] = ld16(qr + 32 * kb + 8 * jq);
    }
  }

  // Physical block of this wavefront's 8 rows of chunk c (rows 8 wave .. +7
  // lie in 16-token tile wave / 2; rows past last_max read last_max's row,
  // chunks past the end included).
  __device__ __forceinline__ int block_of(int c) const {
    const int t = min(CT * c + 16 * (wave >> 1), last_max);
    const int b = bt[t >> LOG2BS];
    return b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
  }

  // this wavefront's share of chunk c's K and V rows into ring slot `slot`
  __device__ __forceinline__ void issue(int c, int blk, int slot) {
    char *dst = ring + slot * CB;
    const int cs = CT * c;
#pragma unroll
    for (int isv = 0; isv < 2; ++isv) {
      const char *base = isv ? vbase : kbase;
      const int64_t sb = isv ? a.v_sb : a.k_sb, st = isv ? a.v_st : a.k_st;
      const char *bb = base + (int64_t)blk * sb * 2;  // uniform block base
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int i = wave * PER + p;
        int r, g;
        Slot::dma_target(isv, i, lane, r, g);
        const int t = min(cs + r, last_max);
        const char *gp = bb + (uint32_t)(((t & (BS - 1)) * (uint32_t)st + 8 * g) * 2);
        __builtin_amdgcn_global_load_lds(gp, lds_addr(dst + isv * HB + 1024 * i), 16, 0, 0);
      }
    }
  }

  // fp8 per-block scales: the key and value scales of chunk c's two tiles'
  // blocks (scalar loads; taken a chunk ahead of their use); 1 without them
  __device__ __forceinline__ void chunk_scales(int c, float *kf, float *vf) const {
    typedef const __attribute__((address_space(4))) float cf;
    kf[0] = kf[1] = vf[0] = vf[1] = 1.0f;
    if (!BSC) return;
    int b[2];
    blocks_of(c, b[0], b[1]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      kf[tt] = ((cf *)(uintptr_t)ksb)[(int64_t)b[tt] * a.num_kv_heads];
      vf[tt] = ((cf *)(uintptr_t)vsb)[(int64_t)b[tt] * a.num_kv_heads];
    }
  }

  // scores and softmax weights of chunk c from the K rows at ks (with the key
  // and value factors kf, vf per 16-token tile when `scaled`)
  __device__ __forceinline__ void qk(int c, const char *ks, u32x4 *phi, u32x4 *plo, bool scaled = false,
                                     const float *kf = nullptr, const float *vf = nullptr) {
    const int cs = CT * c;
    u32x4 kop[2][KS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kb = 0; kb < KS; ++kb) kop[tt][kb] = ld16(ks + koff[kb] + tt * 16 * RB);
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      f32x4 sc[2];
      core[ct].scores(qop[ct], [&](int tt, int kb) { return kop[tt][kb]; }, sc);
      // with the keys split, a wavefront's first chunks may lie past a column's limit
      if (BSC && scaled)
        core[ct].template weights<KSP, true>(sc, cs, last[ct], qk_sc, phi[ct], plo[ct], kf, vf);
      else
        core[ct].template weights<KSP>(sc, cs, last[ct], qk_sc, phi[ct], plo[ct]);
    }
  }
  // output update from the V rows at vs
  __device__ __forceinline__ void pv(const char *vs, const u32x4 *phi, const u32x4 *plo) {
    accumulate_slot_n<NC>(core, phi, plo, vs, [&](int n) { return voff[n]; });
  }
  __device__ __forceinline__ void compute(int c, const char *ks, bool scaled = false, const float *kf = nullptr,
                                          const float *vf = nullptr) {
    u32x4 phi[NC], plo[NC];
    qk(c, ks, phi, plo, scaled, kf, vf);
    pv(ks + HB, phi, plo);
  }

  __device__ void run() {
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) core[ct].reset();
    load_q();
    const int nch = last_max / CT + 1;
    // Chunks c .. c + R - 2 are in flight while chunk c is computed.  Every
    // chunk index issued is loaded (past nch it reloads the last rows into a
    // slot that nobody reads), so each wavefront always has exactly
    // (R - 2) * 2 PER loads outstanding behind the chunk it waits for.
#pragma unroll
    for (int c = 0; c < R - 1; ++c) issue(c, block_of(c), c);
    int nblk = block_of(R - 1);
    int slot = 0, islot = R - 1;  // ring slots of chunk c and of chunk c + R - 1
    for (int c = 0; c < nch; ++c) {
      wait_vm<(R - 2) * 2 * PER>();  // this wavefront's share of chunk c (and the queries before it) has landed
      wg_barrier();                   // every share of chunk c has; everybody is done with chunk c - 1
      __builtin_amdgcn_sched_barrier(0);
      issue(c + R - 1, nblk, islot);
      nblk = block_of(c + R);
      __builtin_amdgcn_sched_barrier(0);
      if (CT * c <= wlast) compute(c, ring + slot * CB);
      __builtin_amdgcn_sched_barrier(0);
      slot = slot + 1 == R ? 0 : slot + 1;
      islot = islot + 1 == R ? 0 : islot + 1;
    }
    wait_vm<0>();  // no load may land after the workgroup's LDS is released
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) core[ct].finish();
  }

  // ---- fp8 caches --------------------------------------------------------
  // Rows come through registers: each 16-byte piece (16 codes) is decoded
  // exactly into two 16-byte granules of the operand type and stored where
  // the 16-bit kernel's DMA would have put them, so the operand reads and the
  // arithmetic are the same.

  // the pieces of rows r0 .. r0 + ROWS - 1 of chunk c, K then V, lane by
  // lane: FP8N<ROWS> pieces per lane; rows of 16-token tile 0 read block b0,
  // those of tile 1 block b1 (rows past last_max read its row)
  template <int ROWS>
  static constexpr int fp8n() { return 2 * ROWS * PPR / 64; }
  template <int ROWS>
  __device__ __forceinline__ void load_fp8(int c, int r0, int b0, int b1, u32x4 *dst) const {
    static_assert((2 * ROWS * PPR) % 64 == 0, "whole pieces per lane");
#pragma unroll
    for (int k = 0; k < fp8n<ROWS>(); ++k) {
      const int idx = lane + 64 * k;
      const int isv = idx / (ROWS * PPR), rem = idx - isv * (ROWS * PPR);
      const int r = r0 + rem / PPR, piece = rem % PPR;
      const int t = min(CT * c + r, last_max);
      const char *base = isv ? vbase : kbase;
      const int64_t sb = isv ? a.v_sb : a.k_sb, st = isv ? a.v_st : a.k_st;
      const int blk = (r & 16) ? b1 : b0;
      const char *gp = base + (int64_t)blk * sb + (uint32_t)((t & (BS - 1)) * (uint32_t)st + 16 * piece);
      // column mode: the tiles of one kv head read the same rows, from L2
      // after the first; the key split reads each row once
      dst[k] = KSP ? ld16_stream(gp) : ld16(gp);
    }
  }
  template <int ROWS>
  __device__ __forceinline__ void stage_fp8(int r0, char *slot, const u32x4 *src) const {
#pragma unroll
    for (int k = 0; k < fp8n<ROWS>(); ++k) {
      const int idx = lane + 64 * k;
      const int isv = idx / (ROWS * PPR), rem = idx - isv * (ROWS * PPR);
      const int r = r0 + rem / PPR, piece = rem % PPR;
      u32x4 o[2];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // codes 4w .. 4w+3 become operand elements 4w .. 4w+3 (exact conversions)
        const uint32_t lo = __is_same(MT, f16_t) ? fp8x2_to_f16x2<false>(src[k][w]) : fp8x2_to_bf16x2<false>(src[k][w]);
        const uint32_t hi = __is_same(MT, f16_t) ? fp8x2_to_f16x2<true>(src[k][w]) : fp8x2_to_bf16x2<true>(src[k][w]);
        o[w >> 1][2 * (w & 1)] = lo;
        o[w >> 1][2 * (w & 1) + 1] = hi;
      }
      char *dst = slot + isv * HB;
#pragma unroll
      for (int h = 0; h < 2; ++h) st16(dst + 16 * Slot::phys(isv, r, 2 * piece + h), o[h]);
    }
  }

  // Column mode, fp8: every wavefront stages its 8 rows of chunk c into the
  // shared ring, a workgroup barrier publishes the chunk (and tells that every
  // wavefront is done with chunk c - 1, so slot c - 1 + R is free), then the
  // wavefront issues its rows of chunk c + 1 and computes chunk c.
  __device__ void run_fp8() {
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) core[ct].reset();
    load_q();
    const int nch = last_max / CT + 1;
    u32x4 rows[fp8n<8>()];
    int blk = block_of(0);
    load_fp8<8>(0, 8 * wave, blk, blk, rows);
    float kf[2], vf[2], nkf[2], nvf[2];  // per-block scales of chunks c and c + 1
    chunk_scales(0, kf, vf);
    int slot = 0;
    for (int c = 0; c < nch; ++c) {
      stage_fp8<8>(8 * wave, ring + slot * CB, rows);
      __syncthreads();  // chunk c staged by every wavefront
      if (c + 1 < nch) {
        blk = block_of(c + 1);
        load_fp8<8>(c + 1, 8 * wave, blk, blk, rows);
      }
      chunk_scales(c + 1, nkf, nvf);
      if (CT * c <= wlast) compute(c, ring + slot * CB, BSC, kf, vf);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        kf[tt] = nkf[tt];
        vf[tt] = nvf[tt];
      }
      slot = slot + 1 == R ? 0 : slot + 1;
    }
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) core[ct].finish();
  }

  // Key split, fp8: the wavefront's chunks wave, wave + 4, ... alternate
  // between its two private slots; the next one is loaded into registers
  // while the current one is computed.
  __device__ void run_split_fp8() {
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) core[ct].reset();
    load_q();
    const int nch = last_max / CT + 1;
    char *mine = ring + wave * 2 * CB;
    u32x4 rows[fp8n<32>()];
    int b0, b1;
    blocks_of(wave, b0, b1);
    load_fp8<32>(wave, 0, b0, b1, rows);
    float kf[2], vf[2], nkf[2], nvf[2];  // per-block scales of chunks c and c + 4
    chunk_scales(wave, kf, vf);
    int k = 0;
    for (int c = wave; c < nch; c += kWaves, ++k) {
      char *slot = mine + (k & 1) * CB;
      stage_fp8<32>(0, slot, rows);
      blocks_of(c + kWaves, b0, b1);
      load_fp8<32>(c + kWaves, 0, b0, b1, rows);  // past the end: the last rows again, unused
      chunk_scales(c + kWaves, nkf, nvf);
      // the transposed reads are inline assembly: keep them after the stores
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      compute(c, slot, BSC, kf, vf);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        kf[tt] = nkf[tt];
        vf[tt] = nvf[tt];
      }
    }
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) core[ct].finish();
  }

  // ---- key split --------------------------------------------------------

  // physical blocks of chunk c's two 16-token tiles (rows past last_max read its row)
  __device__ __forceinline__ void blocks_of(int c, int &b0, int &b1) const {
    const int t0 = min(CT * c, last_max), t1 = min(CT * c + 16, last_max);
    const int x0 = bt[t0 >> LOG2BS], x1 = bt[t1 >> LOG2BS];
    b0 = x0 < 0 ? 0 : (x0 >= a.num_blocks ? a.num_blocks - 1 : x0);
    b1 = x1 < 0 ? 0 : (x1 >= a.num_blocks ? a.num_blocks - 1 : x1);
  }

  // chunk c's K rows (ISV = 0) or V rows (ISV = 1), by this wavefront alone,
  // into the slot at `dst` (K rows at its start, V rows HB bytes in)
  template <int ISV>
  __device__ __forceinline__ void issue_rows(int c, int b0, int b1, char *dst) {
    const int cs = CT * c;
    const char *base = ISV ? vbase : kbase;
    const int64_t sb = ISV ? a.v_sb : a.k_sb, st = ISV ? a.v_st : a.k_st;
#pragma unroll
    for (int i = 0; i < Slot::NLD; ++i) {
      int r, g;
      Slot::dma_target(ISV, i, lane, r, g);
      const int t = min(cs + r, last_max);
      const char *bb = base + (int64_t)((Slot::RPI * i) / 16 ? b1 : b0) * sb * 2;  // uniform block base
      const char *gp = bb + (uint32_t)(((t & (BS - 1)) * (uint32_t)st + 8 * g) * 2);
      __builtin_amdgcn_global_load_lds(gp, lds_addr(dst + ISV * HB + 1024 * i), 16, 0, 0);
    }
  }

  // The wavefront's chunks are wave, wave + 4, ...; two slots, chunk c and
  // chunk c + 4 in the other.  As soon as chunk c's scores are done its K rows
  // take chunk c + 8's, and once its output update is done its V rows do, so
  // about two chunks are in flight at every wait.  Loads are issued in the
  // order K(c), V(c), K(c + 4), V(c + 4), K(c + 8), ...; a chunk index past
  // the end reloads the last rows into a slot nobody reads again, so each wait
  // for K(c) or V(c) has exactly three halves (3 NLD loads) issued after it.
  __device__ void run_split() {
    constexpr int NLD = Slot::NLD;
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) core[ct].reset();
    load_q();
    const int nch = last_max / CT + 1;
    char *mine = ring + wave * 2 * CB;
    int b0, b1;
    blocks_of(wave, b0, b1);
    issue_rows<0>(wave, b0, b1, mine);
    issue_rows<1>(wave, b0, b1, mine);
    blocks_of(wave + kWaves, b0, b1);
    issue_rows<0>(wave + kWaves, b0, b1, mine + CB);
    issue_rows<1>(wave + kWaves, b0, b1, mine + CB);
    blocks_of(wave + 2 * kWaves, b0, b1);  // block ids of chunk c + 8
    int k = 0;
    for (int c = wave; c < nch; c += kWaves, ++k) {
      char *slot = mine + (k & 1) * CB;
      wait_vm<3 * NLD>();  // K(c) (and the queries before it) has landed
      __builtin_amdgcn_sched_barrier(0);
      u32x4 phi[NC], plo[NC];
      qk(c, slot, phi, plo);
      __builtin_amdgcn_sched_barrier(0);
      issue_rows<0>(c + 2 * kWaves, b0, b1, slot);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<3 * NLD>();  // V(c) has landed
      __builtin_amdgcn_sched_barrier(0);
      pv(slot + HB, phi, plo);
      __builtin_amdgcn_sched_barrier(0);
      issue_rows<1>(c + 2 * kWaves, b0, b1, slot);
      blocks_of(c + 3 * kWaves, b0, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm<0>();  // no load may land after the ring is reused or released
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) core[ct].finish();
  }

  // Merge the four wavefronts' (max, sum, output) of every column by
  // log-sum-exp through LDS and write the outputs: wavefront w writes the
  // 16-dim tiles n = w, w + 4, ... of every column.
  template <typename OT>
  __device__ void merge_store() {
    float *pacc = reinterpret_cast<float *>(ring);  // [wave][ct][column][PD]
    float *pml = pacc + kWaves * NC * 16 * PD;      // [wave][ct][column][2]
    __syncthreads();                                // every wavefront is done with the ring
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      float *dst = pacc + ((wave * NC + ct) * 16 + c16) * PD + 4 * jq;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // copy the element out first: a bit cast applied directly to a
          // vector element is lowered as a read of element 0
          const float v = core[ct].acc[n][i];
          w[i] = __builtin_bit_cast(uint32_t, v);
        }
        st16(dst + 16 * n, w);
      }
      if (jq == 0) {
        pml[((wave * NC + ct) * 16 + c16) * 2] = core[ct].m;
        pml[((wave * NC + ct) * 16 + c16) * 2 + 1] = core[ct].l;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      float m[kWaves], f[kWaves];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        m[w] = pml[((w * NC + ct) * 16 + c16) * 2];
        M = fmaxf(M, m[w]);
      }
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        f[w] = fast_exp2(m[w] - M);  // 0 for a wavefront that saw none of this column's positions
        L += f[w] * pml[((w * NC + ct) * 16 + c16) * 2 + 1];
      }
      const bool z = last[ct] < 0;
      const float inv = v_sc / L;
      const int64_t off = (int64_t)row[ct] * a.o_sn + (int64_t)head[ct] * a.o_sh + 4 * jq;
#pragma unroll
      for (int n = wave; n < NT; n += kWaves) {
        float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const u32x4 x = ld16(pacc + ((w * NC + ct) * 16 + c16) * PD + 16 * n + 4 * jq);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t xi = x[i];
            o[i] += f[w] * __builtin_bit_cast(float, xi);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = z ? 0.0f : o[i] * inv;
        if (valid[ct]) store4<OT>(a.out, off + 16 * n, o);
      }
    }
  }

  __device__ void merge_write() {
    if (a.out_f32)
      merge_store<f32_t>();
    else
      merge_store<MT>();
  }

  template <typename OT>
  __device__ __forceinline__ void store(int ct, bool zero) const {
    const float inv = v_sc / core[ct].l;
    const bool z = zero || last[ct] < 0;
    const int64_t off = (int64_t)row[ct] * a.o_sn + (int64_t)head[ct] * a.o_sh + 4 * jq;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = z ? 0.0f : core[ct].acc[n][i] * inv;
      store4<OT>(a.out, off + 16 * n, o);
    }
  }

  // outputs of the valid columns (zeros when `zero`, or for a row before position 0)
  __device__ void write_out(bool zero) const {
#pragma unroll
    for (int ct = 0; ct < NC; ++ct) {
      if (!valid[ct]) continue;
      if (a.out_f32)
        store<f32_t>(ct, zero);
      else
        store<MT>(ct, zero);
    }
  }
};

template <typename MT, typename KVT, int D, int BS, int NC, bool KSP, bool BSC = false>
__global__ void __launch_bounds__(64 * kWaves, KSP ? 1 : 2) prefill_mfma(const PrefillArgs a) {
  typedef PrefillTile<MT, KVT, D, BS, NC, KSP, BSC> Tile;
  __shared__ __attribute__((aligned(1024))) char lds[Tile::kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  TileOrder order;
  order.init(a, lane);
  int seq, tile;
  if constexpr (KSP) {
    // Key split (about one tile per sequence and kv head): persistent
    // workgroups, one per CU, take the (tile, kv head) pairs in the tiles'
    // order, all kv heads of a tile in a row, longest contexts first.  The
    // first pairs are dealt one per workgroup; with a pair counter each
    // workgroup then takes the next pair as it frees up (longest processing
    // time first), else it takes every gridDim.x-th pair.  Every workgroup's
    // last take returns a pair past the end, so the takes number exactly n
    // (the grid never exceeds n) and the one that returns n - 1 is the last:
    // it resets the counter for the next call.
    const int n = (order.ranked ? order.total : a.tile_slots) * a.num_kv_heads;
    __shared__ int next_pair;
    for (int x = blockIdx.x; x < n;) {
      const int t = x / a.num_kv_heads, kvh = x - t * a.num_kv_heads;
      const bool found = order.find(a, t, lane, seq, tile);  // unranked batches: none past the last tile
      if (!found && a.pair_counter == nullptr) break;      // (with a counter, keep taking to the end)
      if (found) {
        Tile tl(a, lds, lane, wave);
        if (tl.setup(seq, tile, kvh)) {
          if constexpr (Tile::kFp8)
            tl.run_split_fp8();
          else
            tl.run_split();
          tl.merge_write();
        } else if (wave == 0) {
          tl.write_out(true);
        }
      }
      __syncthreads();  // the merge's reads of the ring are done before the next tile's loads
      if (a.pair_counter == nullptr) {
        x += gridDim.x;
        continue;
      }
      if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(a.pair_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == n - 1) __hip_atomic_store(a.pair_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        next_pair = (int)gridDim.x + old;
      }
      __syncthreads();
      x = next_pair;
    }
  } else {
    // Workgroups are dealt to the 8 XCDs round-robin; number them so that the
    // tiles of one kv head, which read the same K/V rows, share an XCD's L2.
    const int nb = gridDim.x, b = blockIdx.x;
    const int bx = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
    const int kvh = bx / a.tile_slots;
    if (kvh >= a.num_kv_heads) return;
    if (!order.find(a, bx - kvh * a.tile_slots, lane, seq, tile)) return;  // the same for all four wavefronts
    Tile tl(a, lds, lane, wave);
    if (!tl.setup(seq, tile, kvh)) {
      tl.write_out(true);
      return;
    }
    if constexpr (Tile::kFp8)
      tl.run_fp8();
    else
      tl.run();
    tl.write_out(false);
  }
}

template <typename MT, typename KVT, int D, int BS, bool BSC>
hipError_t launch_nc(const PrefillArgs &a, hipStream_t stream) {
  const int64_t n = (int64_t)a.tile_slots * a.num_kv_heads;
  const dim3 grid((unsigned)(a.key_split ? min((int64_t)a.persistent_wgs, n) : (n + 7) / 8 * 8)),
      block(64 * kWaves);
  if (a.key_split) {
    if (a.tile_cols == 32)
      hipLaunchKernelGGL((prefill_mfma<MT, KVT, D, BS, 2, true, BSC>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_mfma<MT, KVT, D, BS, 1, true, BSC>), grid, block, 0, stream, a);
  } else {
    if (a.tile_cols == 32 * kWaves)
      hipLaunchKernelGGL((prefill_mfma<MT, KVT, D, BS, 2, false, BSC>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_mfma<MT, KVT, D, BS, 1, false, BSC>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

template <typename MT, typename KVT, int D, bool BSC>
hipError_t launch_bs(const PrefillArgs &a, hipStream_t stream) {
  return a.block_size == 16 ? launch_nc<MT, KVT, D, 16, BSC>(a, stream) : launch_nc<MT, KVT, D, 32, BSC>(a, stream);
}

template <typename MT, typename KVT>
hipError_t launch_d(const PrefillArgs &a, hipStream_t stream) {
  if constexpr (__is_same(KVT, fp8_t)) {  // per-block scales: their own variant
    if (a.k_block_scale != nullptr) {
      switch (a.head_dim) {
        case 64: return launch_bs<MT, KVT, 64, true>(a, stream);
        case 128: return launch_bs<MT, KVT, 128, true>(a, stream);
      }
      return hipErrorInvalidValue;
    }
  }
  switch (a.head_dim) {
    case 64: return launch_bs<MT, KVT, 64, false>(a, stream);
    case 128: return launch_bs<MT, KVT, 128, false>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool prefill_supported(int kv_kind, int head_dim) {
  return (kv_kind == KV_F16 || kv_kind == KV_BF16 || kv_kind == KV_FP8) && (head_dim == 64 || head_dim == 128);
}

// Tile shape.  Steps that average at most 32 columns per sequence (a few
// query rows, verification-sized) split the keys of a 16- or 32-column tile
// over the four wavefronts; larger steps give each wavefront its own columns:
// 32 when the sequences average at least two such tiles' worth (each K/V
// operand read from LDS then feeds twice the arithmetic), else 16.
void prefill_plan(int64_t num_rows, int64_t num_seqs, int group, int &tile_cols, int &key_split) {
  const int64_t cols = num_rows * group;
  key_split = cols <= 32 * num_seqs;
  if (key_split)
    tile_cols = cols <= 16 * num_seqs ? 16 : 32;
  else
    tile_cols = cols >= 2 * 32 * kWaves * num_seqs ? 32 * kWaves : 16 * kWaves;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  switch (a.kv_kind) {
    case KV_F16: return launch_d<f16_t, f16_t>(a, stream);
    case KV_BF16: return launch_d<bf16_t, bf16_t>(a, stream);
    case KV_FP8:
      if (a.q_kind == KV_F16) return launch_d<f16_t, fp8_t>(a, stream);
      if (a.q_kind == KV_BF16) return launch_d<bf16_t, fp8_t>(a, stream);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
