// Paged decode for grouped-query heads on the matrix cores (MFMA).
//
// When G = num_heads / num_kv_heads query heads read one KV head, the scores
// of a chunk of tokens and the output update are small dense contractions:
//   S^T[t][h] = sum_d K[t][d] q[h][d]        (tokens x heads, over head_dim)
//   O^T[d][h] += sum_t V[t][d] P[h][t]       (head_dim x heads, over tokens)
// Both run as v_mfma_f32_16x16x32 (f16 or bf16 operands, fp32 accumulation),
// with the G heads padded to the 16 columns of the instruction.  Everything
// else -- the block-table walk, the per-wavefront balanced split and the
// log-sum-exp merge -- is the same as on the vector-ALU path (pa_sched.h), and
// follows the same pages: logical-to-physical translation of page
// "vLLM框架中的KV cache优化与PagedAttention机制详解" (section 5.1), address rule of
// page "Paged KVCache：大模型推理显存管理优化方案" (section 2.3), per-block scores
// accumulated across blocks as page "vLLM推理引擎架构：PagedAttention机制与高吞吐推理"
// (section 2.3) describes.
//
// Lane layouts (v_mfma_f32_16x16x32: lane l holds row l % 16 and the 8
// consecutive k-indices 8 * (l / 16) .. +7 of A; column l % 16 and the same
// k-indices of B; rows 4 * (l / 16) + i, i < 4, column l % 16 of C):
//   QK  A = K tile (16 tokens x 32 dims): lane (t, j) loads 16 bytes of token
//       t's row at dims 32 kb + 8 j -- for each k-step kb the 16 rows are read
//       in 64-byte pieces, so every instruction is coalesced;
//       B = q^T: lane (h, j) holds q[h][32 kb + 8 j ..]; zero for h >= G.
//       The output gives lane (h, j) the scores of head h for tokens 4 j + i.
//   PV  A = V^T tile (16 dims x 32 tokens), B = P^T (32 tokens x 16 heads).
//       The chunk's 32 tokens enter the contraction in the order
//       tau(j, i) = 4 j + i (i < 4), 16 + 4 j + i - 4 (i >= 4), which is
//       exactly the 8 scores lane (h, j) already holds from the two QK tiles,
//       so P needs no exchange between lanes.  V rows are staged through LDS
//       (one 32-row buffer per wavefront) and read back transposed.
//       The output gives lane (h, j) dims 16 n + 4 j + i of head h -- the same
//       head as its softmax state, so the rescale by exp2(m_old - m_new) is
//       per lane.
//   P is split as P = hi + lo in the operand type (f16 or bf16) and both parts
//   are multiplied in, so the weights carry ~16 more bits than one rounding
//   would give (a single bf16 rounding of the weights alone would cost more
//   than the fp32-output error budget).
// K and V rows pass through LDS, so the next chunk's loads go out as soon as
// this chunk's rows are staged, before any of its arithmetic.  fp8 caches are decoded exactly into the
// query's 16-bit type on the way (every e4m3fn value is representable).
#include "mfma_core.h"
#include "pa_sched.h"

namespace pa {

namespace {

using namespace mfma;

constexpr int kWavesPerWG = 4;

// A 16-byte piece of a cache row (8 16-bit elements or 16 fp8 codes) and its
// conversion to the operand type.
template <typename KVT, typename MT> struct Piece {
  static constexpr int kElems = 8;
  __device__ static void to_op(u32x4 r, u32x4 *o) { o[0] = r; }
};
template <typename MT> struct Piece<fp8_t, MT> {
  static constexpr int kElems = 16;
  __device__ static void to_op(u32x4 r, u32x4 *o) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // codes 4w .. 4w+3 become operand elements 4w .. 4w+3 (exact conversions)
      const uint32_t lo = __is_same(MT, f16_t) ? fp8x2_to_f16x2<false>(r[w]) : fp8x2_to_bf16x2<false>(r[w]);
      const uint32_t hi = __is_same(MT, f16_t) ? fp8x2_to_f16x2<true>(r[w]) : fp8x2_to_bf16x2<true>(r[w]);
      o[w >> 1][2 * (w & 1)] = lo;
      o[w >> 1][2 * (w & 1) + 1] = hi;
    }
  }
};

// The arithmetic of one wavefront on one (sequence, kv head) segment, whatever
// brings the chunk's rows into LDS: scores, online softmax, output update and
// the segment's epilogue.
template <typename MT, int D, int G>
struct MfmaMath : MfmaCore<MT, D> {
  using Core = MfmaCore<MT, D>;
  using Core::acc;
  using Core::c16;
  using Core::j;
  using Core::l;
  using Core::m;
  static constexpr int KS = Core::KS;
  static constexpr int NT = Core::NT;
  static_assert(G >= 2 && G <= 16, "group must fit the 16 columns");

  const DecodeArgs &a;
  ItemScale isc;  // the segment's scales (the launch's, or its fp8 kv head's)

  __device__ MfmaMath(const DecodeArgs &args, int lane) : Core(lane), a(args), isc{args.qk_scale_log2, args.v_scale} {}

  // online softmax for head c16 (tokens past `last` masked)
  __device__ __forceinline__ void weights(const f32x4 *sc, int cs, int last, u32x4 &phi, u32x4 &plo) {
    Core::weights(sc, cs, last, isc.qk, phi, plo);
  }
  // the same with a key and a value factor per 16-token tile
  __device__ __forceinline__ void weights(const f32x4 *sc, int cs, int last, const float *kf, const float *vf,
                                          u32x4 &phi, u32x4 &plo) {
    Core::template weights<false, true>(sc, cs, last, isc.qk, phi, plo, kf, vf);
  }

  __device__ void write_out(int s, int kvh) const {
    if (c16 >= G) return;
    const float inv = isc.v / l;
    const int64_t row = o_row(a, s) + (int64_t)(kvh * G + c16) * a.o_sh;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[n][i] * inv;
      if (a.out_f32)
        store4<f32_t>(a.out, row + 16 * n + 4 * j, o);
      else
        store4<MT>(a.out, row + 16 * n + 4 * j, o);
    }
  }

  __device__ void write_partial(int64_t slot) const {
    if (c16 >= G) return;
    const int64_t pacc = slot_acc<G, D>(slot) + c16 * D;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[n][i];
      store_shared4(a, pacc + 16 * n + 4 * j, o);
    }
    if (j == 0) {
      const int64_t pml = slot_ml<G>(slot);
      store_shared_ml(a, pml + 2 * c16, m);
      store_shared_ml(a, pml + 2 * c16 + 1, l);
    }
  }
};

// ---------------------------------------------------------------------------
// fp8 caches: rows are loaded into registers, decoded, and staged in LDS as
// the operand type (the loads of chunk c+1 are in flight while chunk c is
// computed).
// BSC: one scale per (block, kv head) (a variant of its own, so that the
// other launches carry none of its work)
template <typename KVT, typename MT, int D, int G, int BS, bool BSC = false>
struct MfmaRegSeg : MfmaMath<MT, D, G> {
  using Math = MfmaMath<MT, D, G>;
  using Math::a;
  using Math::c16;
  using Math::j;
  static constexpr int KS = Math::KS;
  static constexpr int NT = Math::NT;
  static constexpr int LOG2BS = BS == 16 ? 4 : 5;
  static constexpr int EB = Elem<KVT>::kBytes;
  static constexpr int PE = Piece<KVT, MT>::kElems;  // elements per 16-byte piece
  static constexpr int LPR = D / PE;                  // lanes per cache row
  static constexpr int RPI = 64 / LPR;                // rows per load instruction
  static constexpr int NLD = CT / RPI;                // load instructions per chunk (K or V)
  // halves per staged row; the paddings put the rows that one LDS access
  // touches on distinct banks: 16 consecutive rows for the 16-byte K operand
  // reads (a 4-bank shift per row), 4 consecutive rows for the transposed V
  // reads (an 8-bank shift per row)
  static constexpr int KSTRIDE = D + 8;
  static constexpr int VSTRIDE = D + 16;
  static constexpr int kLdsBytes = 2 * CT * (KSTRIDE + VSTRIDE);
  static_assert(RPI <= 16 && 16 % RPI == 0, "a load instruction stays inside one 16-token tile");

  const int lrow, lpiece;  // row of a load instruction and 16-byte piece of the row this lane loads
  uint16_t *ks, *vs;       // this wavefront's LDS stages [CT][KSTRIDE], [CT][VSTRIDE], operand type

  __device__ MfmaRegSeg(const DecodeArgs &args, int ln, char *lds)
      : Math(args, ln), lrow(ln / LPR), lpiece(ln % LPR), ks(reinterpret_cast<uint16_t *>(lds)),
        vs(reinterpret_cast<uint16_t *>(lds) + CT * KSTRIDE) {}

  // block ids of the chunk's two 16-token tiles (loads past `last` read its block)
  __device__ __forceinline__ void fetch_blocks(const_i32 *bt, int cs, int last, int *blk) const {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      int b = bt[min(cs + 16 * tt, last) >> LOG2BS];
      blk[tt] = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
    }
  }

  // Whole cache rows: instruction i reads rows RPI i .. RPI i + RPI - 1 of the
  // chunk, LPR lanes per row, 16 bytes each -- every row a contiguous run.
  __device__ __forceinline__ void issue(const char *base, int64_t sb, int64_t st, int cs, int last, const int *blk,
                                        u32x4 *dst) const {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int row = RPI * i + lrow;
      const int t = min(cs + row, last);
      const char *bb = base + (int64_t)blk[(RPI * i) / 16] * sb * EB;  // uniform block base
      dst[i] = ld16_stream(bb + (uint32_t)(((t & (BS - 1)) * (uint32_t)st + lpiece * PE) * EB));
    }
  }

  // the chunk's rows into an LDS stage, as the operand type
  template <int STRIDE>
  __device__ __forceinline__ void stage(uint16_t *dst, const u32x4 *r) const {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      u32x4 o[PE / 8];
      Piece<KVT, MT>::to_op(r[i], o);
#pragma unroll
      for (int h = 0; h < PE / 8; ++h) st16(dst + (RPI * i + lrow) * STRIDE + lpiece * PE + 8 * h, o[h]);
    }
  }

  __device__ __forceinline__ u32x4 k_operand(int tt, int kb) const {
    return *reinterpret_cast<const u32x4 *>(ks + (16 * tt + c16) * KSTRIDE + 32 * kb + 8 * j);
  }

  // ds_read_b64_tr_b16 hands lane i of a 16-lane group the elements
  // M[4 r + i / 4][i % 4], r < 4, where M[k] are the four 16-bit values at lane
  // k's address.  Lane k of quarter j therefore points at row tau(j, 4 h + k / 4)
  // (h = which half of the operand), columns 16 n + 4 (k % 4) .. +3: lane i
  // receives column 16 n + i of the four rows, in the contraction's order.
  __device__ __forceinline__ u32x4 vt_operand(int n) const {
    const int col = 16 * n + 4 * (c16 & 3);
    const uint16_t *r0 = vs + (4 * j + (c16 >> 2)) * VSTRIDE + col;       // tokens 4 j .. 4 j + 3
    const uint16_t *r1 = vs + (16 + 4 * j + (c16 >> 2)) * VSTRIDE + col;  // tokens 16 + 4 j ..
    return read_tr(r0, r1);
  }

  // where a segment's rows live
  struct Ptrs {
    const_i32 *bt;
    const char *kb, *vb;
    int last;
    const float *ksb, *vsb;  // per-block scales: this layer's and kv head's (stride num_kv_heads per block), or null
  };
  __device__ __forceinline__ Ptrs ptrs(const SegInfo &g) const {
    Ptrs p;
    p.bt = as_const(a.block_tables) + (int64_t)seq_of(a, g.s) * a.bt_ss;
    p.kb = reinterpret_cast<const char *>(a.k_cache) + (k_layer(a, g.s) + (int64_t)g.kvh * a.k_sh) * EB;
    p.vb = reinterpret_cast<const char *>(a.v_cache) + (v_layer(a, g.s) + (int64_t)g.kvh * a.v_sh) * EB;
    p.last = g.t_hi - 1;
    p.ksb = p.vsb = nullptr;
    if (BSC) {
      const int64_t o = (int64_t)layer_of(a, g.s) * a.num_blocks * a.num_kv_heads + g.kvh;
      p.ksb = a.k_block_scale + o;
      p.vsb = a.v_block_scale + o;
    }
    return p;
  }
  // per-block scales: the key and value scales of the chunk's two tiles'
  // blocks (scalar loads, a chunk ahead of their use); 1 without them
  __device__ __forceinline__ void fetch_scales(const float *ksb, const float *vsb, const int *blk, float *kf,
                                               float *vf) const {
    typedef const __attribute__((address_space(4))) float cf;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      kf[tt] = vf[tt] = 1.0f;
      if (BSC) {
        kf[tt] = ((cf *)(uintptr_t)ksb)[(int64_t)blk[tt] * a.num_kv_heads];
        vf[tt] = ((cf *)(uintptr_t)vsb)[(int64_t)blk[tt] * a.num_kv_heads];
      }
    }
  }
  // q^T operand: lane (h, j) holds q[h][32 kb + 8 j ..], zeros for padding heads
  __device__ __forceinline__ void load_q(const SegInfo &g, u32x4 *dst) const {
    const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) + q_row(a, g.s) +
                           (int64_t)(g.kvh * G + (c16 < G ? c16 : 0)) * a.q_sh;
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) {
      dst[kb] = ld16(qrow + 32 * kb + 8 * j);
      if (c16 >= G) dst[kb] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // pipeline state carried from one segment into the next
  u32x4 qop[KS];
  int blk[2];
  float kf[2], vf[2];  // the current chunk's tiles' key and value block scales (1 without per-block scales)
  u32x4 kr[NLD], vr[NLD];

  __device__ void begin(const SegInfo &g, const Walker &) { begin(g); }
  __device__ void publish(const SegInfo &g, const Split &sp) {
    finish_partial<MT, G, D>(a, g.s, g.kvh, g.a0, g.n, sp, 16 * j + c16);
  }
  __device__ void end() {}

  __device__ void begin(const SegInfo &g) {
    const Ptrs p = ptrs(g);
    load_q(g, qop);
    fetch_blocks(p.bt, g.t_lo, p.last, blk);
    if constexpr (BSC) fetch_scales(p.ksb, p.vsb, blk, kf, vf);
    __builtin_amdgcn_sched_barrier(0);
    issue(p.kb, a.k_sb, a.k_st, g.t_lo, p.last, blk, kr);
    __builtin_amdgcn_sched_barrier(0);
    issue(p.vb, a.v_sb, a.v_st, g.t_lo, p.last, blk, vr);
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ void run(const SegInfo &g, const SegInfo &nx, bool has) {
    Math::reset();
    if (g.t_hi <= g.t_lo) {  // only if context_lens changed under the launch
      if (has) begin(nx);
      return;
    }
    Math::isc = seg_scale<KVT>(a, g.s, g.kvh);
    const Ptrs p = ptrs(g);
    // the chunk after this segment's last one: the next segment's first (or,
    // for the range's last segment, this last chunk again -- a cache hit, unused)
    const Ptrs pn = has ? ptrs(nx) : p;
    u32x4 qn[KS];
    load_q(has ? nx : g, qn);

    const int nch = (g.t_hi - g.t_lo + CT - 1) / CT;
    int cs = g.t_lo;
    for (int c = 0; c < nch; ++c) {
      const bool lastc = c + 1 == nch;
      const int cn = lastc ? (has ? nx.t_lo : cs) : cs + CT;
      const_i32 *btn = lastc ? pn.bt : p.bt;
      const char *kbn = lastc ? pn.kb : p.kb;
      const char *vbn = lastc ? pn.vb : p.vb;
      const int lastn = lastc ? pn.last : p.last;
      int nblk[2];
      fetch_blocks(btn, cn, lastn, nblk);
      float nkf[2], nvf[2];
      if constexpr (BSC) fetch_scales(lastc ? pn.ksb : p.ksb, lastc ? pn.vsb : p.vsb, nblk, nkf, nvf);
      __builtin_amdgcn_sched_barrier(0);

      // this chunk's K and V rows to LDS, then the next chunk's loads into the
      // freed registers: a whole chunk stays in flight while this one is computed
      stage<KSTRIDE>(ks, kr);
      __builtin_amdgcn_sched_barrier(0);
      issue(kbn, a.k_sb, a.k_st, cn, lastn, nblk, kr);
      __builtin_amdgcn_sched_barrier(0);
      stage<VSTRIDE>(vs, vr);
      __builtin_amdgcn_sched_barrier(0);
      issue(vbn, a.v_sb, a.v_st, cn, lastn, nblk, vr);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 sc[2];
      Math::scores(qop, [&](int tt, int kb) { return k_operand(tt, kb); }, sc);
      u32x4 phi, plo;
      if constexpr (BSC)
        Math::weights(sc, cs, p.last, kf, vf, phi, plo);
      else
        Math::weights(sc, cs, p.last, phi, plo);
      Math::accumulate(phi, plo, [&](int n) { return vt_operand(n); });
      cs = cn;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        blk[tt] = nblk[tt];
        if constexpr (BSC) {
          kf[tt] = nkf[tt];
          vf[tt] = nvf[tt];
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) qop[kb] = qn[kb];
    Math::finish();
  }
};

// ---------------------------------------------------------------------------
// 16-bit caches: rows go from HBM straight into LDS (global_load_lds_dwordx4,
// no registers on the way), into a per-wavefront ring of four half-chunk
// slots -- K and V rows of two chunks -- and two query slots.  While chunk c
// is computed the loads of V(c+1) and K(c+2) go out, so about two chunks of
// rows are in flight at every wait.  The waits are explicit (vmcnt): every
// load step issues the same number of instructions (past the range's end it
// reloads its last chunk into a slot nobody reads), so waiting until at most
// kAhead instructions are outstanding guarantees the awaited slot has landed;
// occasional query loads only make that wait stricter.
//
// Rows sit in a slot in the swizzled placement of RowSlot (mfma_core.h).  A
// DMA instruction fills 1 KB of LDS in lane order, so each lane fetches the
// global granule that belongs at its LDS position.
template <typename MT, int D, int G, int BS, bool APPEND = false>
struct MfmaRingSeg : MfmaMath<MT, D, G> {
  using Math = MfmaMath<MT, D, G>;
  using Math::a;
  using Math::c16;
  using Math::j;
  static constexpr int KS = Math::KS;
  static constexpr int NT = Math::NT;
  static constexpr int LOG2BS = BS == 16 ? 4 : 5;
  using Slot = RowSlot<D>;
  static constexpr int RB = Slot::RB;                       // bytes per cache row
  static constexpr int HB = Slot::HB;                       // bytes of a half-chunk slot
  static constexpr int NLD = Slot::NLD;                     // DMA instructions per half-chunk
  static constexpr int RPI = Slot::RPI;                     // rows per DMA instruction
  static constexpr int QB = G * RB > 1024 ? G * RB : 1024;  // bytes of a query slot
  static constexpr int kLdsBytes = 4 * HB + 2 * QB;
  static constexpr int kAhead = 3 * NLD;  // instructions issued after the half-chunk a wait is for
  static constexpr int kNontemporal = 2;  // cache-policy operand of the DMA: streaming (nt)
  static_assert(kLdsBytes * kWavesPerWG <= 160 * 1024, "ring fits the LDS of a CU");

  typedef __attribute__((address_space(3))) void lds_void;
  __device__ static lds_void *lds_addr(char *p) { return (lds_void *)p; }

  struct Src {
    const char *base;  // cache + kv head offset
    int blk0, blk1;    // block ids of the chunk's two 16-token tiles
    int cs, last;      // first token of the chunk, last token of its segment
    int nrow;          // fused step, an item's last segment: (sequence * kv heads + kv head) of the new token's
                       // row, read for token `last`; else -1
  };

  char *ring;  // this wavefront's LDS: K0 V0 K1 V1 (HB each), Q0 Q1 (QB each)
  const int lane;
  int koff[KS];  // lane byte offset of the K operand of k-step kb, tile 0
  int voff[NT];  // lane byte offset of the first half of the V^T operand of tile n

  Split sp;  // the launch's split of the work over the workers

  // load cursor: the worker's chunk stream, two chunks ahead of the arithmetic
  Walker lw;
  SegInfo ls;
  bool lhas;
  int lcs, llast;  // next chunk of ls to load; last token of ls
  const_i32 *lbt;
  const char *lkb, *lvb;  // K / V rows of ls: its layer's cache at its kv head
  int lnrow;  // fused step, ls the last segment of its item: (sequence * kv heads + kv head) of the new rows; else -1
  int nblk[2];  // block ids of chunk lcs
  int lord;     // non-empty segments whose query has been loaded
  Src vpend;    // the chunk whose V rows go out next
  Walker cw;    // the arithmetic's own walk over the same segments
  int ccnt;     // chunks consumed by the arithmetic (ring slot parity)
  int cord;     // non-empty segments consumed by the arithmetic (query slot parity)
  u32x4 qop[KS];

  __device__ MfmaRingSeg(const DecodeArgs &args, int ln, char *lds)
      : Math(args, ln), ring(lds), lane(ln), lw(args), cw(args) {
#pragma unroll
    for (int kb = 0; kb < KS; ++kb) koff[kb] = Slot::k_off(c16, j, kb);
#pragma unroll
    for (int n = 0; n < NT; ++n) voff[n] = Slot::v_off(c16, j, n);
  }

  __device__ __forceinline__ void fetch_blocks(int cs, int last, int *blk) const {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      int b = lbt[min(cs + 16 * tt, last) >> LOG2BS];
      blk[tt] = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
    }
  }

  // the 32 rows of one chunk's K or V into a ring slot; in a fused step the
  // chunk that holds an item's last token takes that row from the new rows
  template <bool ISV>
  __device__ __forceinline__ void dma(const Src &src, int64_t sb, int64_t st, char *slot) const {
    // in a fused step the chunk that holds an item's new token takes that row's
    // granules from the new rows: a per-lane address choice, no second loop
    const bool redirect = APPEND && uniform(src.nrow >= 0 && src.cs + CT > src.last);
    const char *nb = nullptr;
    if (APPEND) {
      const int s = src.nrow / a.num_kv_heads, kvh = src.nrow - (src.nrow / a.num_kv_heads) * a.num_kv_heads;
      nb = reinterpret_cast<const char *>(ISV ? a.v_new : a.k_new) +
           ((int64_t)s * (ISV ? a.vn_ss : a.kn_ss) + (int64_t)kvh * (ISV ? a.vn_sh : a.kn_sh)) * 2;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      int r, g;
      Slot::dma_target(ISV, i, lane, r, g);
      const int t = min(src.cs + r, src.last);
      const int blk = (RPI * i) / 16 ? src.blk1 : src.blk0;
      const char *bb = src.base + (int64_t)blk * sb * 2;  // uniform block base
      const char *gp = bb + (uint32_t)(((t & (BS - 1)) * (uint32_t)st + 8 * g) * 2);
      if (APPEND && redirect)  // a scalar branch around the choice only: the DMA instruction is the same
        gp = reinterpret_cast<const char *>(t == src.last ? (uintptr_t)(nb + 16 * g) : (uintptr_t)gp);
      __builtin_amdgcn_global_load_lds(gp, lds_addr(slot + 1024 * i), 16, 0, kNontemporal);
    }
  }

  // the G query rows of segment g into a query slot (rows past G in a 1 KB
  // slot reload row 0)
  __device__ __forceinline__ void dma_q(const SegInfo &g, char *slot) const {
#pragma unroll
    for (int i = 0; i < QB / 1024; ++i) {
      const int b = 1024 * i + 16 * lane;
      const int h = b / RB < G ? b / RB : 0;
      const char *gp = reinterpret_cast<const char *>(a.q) +
                       (q_row(a, g.s) + (int64_t)(g.kvh * G + h) * a.q_sh + (b % RB) / 2) * 2;
      __builtin_amdgcn_global_load_lds(gp, lds_addr(slot + 1024 * i), 16, 0, 0);
    }
  }

  __device__ __forceinline__ void next_load_seg() {
    do {
      lhas = lw.next(ls);
    } while (lhas && ls.t_hi <= ls.t_lo);
    if (lhas) {
      lbt = as_const(a.block_tables) + (int64_t)seq_of(a, ls.s) * a.bt_ss;
      lkb = reinterpret_cast<const char *>(a.k_cache) + (k_layer(a, ls.s) + (int64_t)ls.kvh * a.k_sh) * 2;
      lvb = reinterpret_cast<const char *>(a.v_cache) + (v_layer(a, ls.s) + (int64_t)ls.kvh * a.v_sh) * 2;
      lnrow = APPEND && ls.u_hi == ls.n && append_writes(a, ls.s) ? ls.s * a.num_kv_heads + ls.kvh : -1;
      lcs = ls.t_lo;
      llast = ls.t_hi - 1;
      fetch_blocks(lcs, llast, nblk);
    }
  }

  // K rows of the cursor's next chunk (its query first, at a segment's start)
  // into K slot `par`
  __device__ __forceinline__ void issue_k(int par) {
    char *slot = ring + par * 2 * HB;
    if (lhas) {
      if (lcs == ls.t_lo) {
        dma_q(ls, ring + 4 * HB + (lord & 1) * QB);
        ++lord;
      }
      const Src k{lkb, nblk[0], nblk[1], lcs, llast, lnrow};
      vpend = Src{lvb, nblk[0], nblk[1], lcs, llast, lnrow};
      dma<false>(k, a.k_sb, a.k_st, slot);
      lcs += CT;
      if (lcs < ls.t_hi)
        fetch_blocks(lcs, llast, nblk);
      else
        next_load_seg();
    } else {
      dma<false>(vpend, a.v_sb, a.v_st, slot);  // nothing left: reload rows into a slot nobody reads
    }
  }

  // V rows of the chunk whose K rows went out last, into V slot `par`
  __device__ __forceinline__ void issue_v(int par) { dma<true>(vpend, a.v_sb, a.v_st, ring + (par * 2 + 1) * HB); }

  // Start on this worker's range [b, e); false if there is nothing to do.
  __device__ bool start(const Split &split, const Windows &first, int64_t b, int64_t e) {
    sp = split;
    ccnt = cord = lord = 0;
    vpend = Src{reinterpret_cast<const char *>(a.v_cache), 0, 0, 0, 0, -1};  // reloaded when there is nothing left
    if (!cw.init(first, b, e, lane)) return false;
    lw = cw;
    next_load_seg();
    issue_k(0);
    issue_v(0);
    issue_k(1);
    return true;
  }

  // the arithmetic's next segment
  __device__ bool next_segment(SegInfo &g) { return cw.next(g); }

  // Count a cut segment's partial.  Its write-through stores must be
  // complete first, and a vmcnt count cannot tell stores from the DMA loads
  // issued after them (loads and stores may complete out of order), so this
  // waits for everything outstanding.
  __device__ void publish(const SegInfo &g) { finish_partial<MT, G, D>(a, g.s, g.kvh, g.a0, g.n, sp, lane); }

  // no DMA may land after the wavefront's LDS is released
  __device__ void end() { wait_vm<0>(); }

  __device__ void run(const SegInfo &g) {
    Math::reset();
    if (g.t_hi <= g.t_lo) return;  // only if context_lens changed under the launch
    const int last = g.t_hi - 1;
    const int nch = (g.t_hi - g.t_lo + CT - 1) / CT;
    int cs = g.t_lo;
    for (int c = 0; c < nch; ++c) {
      const int par = ccnt & 1;
      issue_v(par ^ 1);  // V(c+1)
      wait_vm<kAhead>();  // K rows of this chunk (and, before them, the segment's query) have landed
      __builtin_amdgcn_sched_barrier(0);
      if (c == 0) {
        const char *qs = ring + 4 * HB + (cord & 1) * QB + (c16 < G ? c16 : 0) * RB;
#pragma unroll
        for (int kb = 0; kb < KS; ++kb) {
          qop[kb] = ld16(qs + (4 * kb + j) * 16);
          if (c16 >= G) qop[kb] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      const char *ks = ring + par * 2 * HB;
      u32x4 kop[2][KS];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int kb = 0; kb < KS; ++kb) kop[tt][kb] = ld16(ks + koff[kb] + tt * 16 * RB);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 sc[2];
      Math::scores(qop, [&](int tt, int kb) { return kop[tt][kb]; }, sc);
      __builtin_amdgcn_sched_barrier(0);
      issue_k(par);  // K(c+2), into the slot just read
      __builtin_amdgcn_sched_barrier(0);
      u32x4 phi, plo;
      Math::weights(sc, cs, last, phi, plo);
      wait_vm<kAhead>();  // V rows of this chunk
      __builtin_amdgcn_sched_barrier(0);
      Math::accumulate_slot(phi, plo, ring + (par * 2 + 1) * HB, [&](int n) { return voff[n]; });
      __builtin_amdgcn_sched_barrier(0);
      cs += CT;
      ++ccnt;
    }
    ++cord;
    Math::finish();
  }
};

// One worker of the ring kernel: its range, segment by segment; the
// segment owns both walks over it (loads ahead, arithmetic behind).
template <typename MT, int G, int D, class Seg, bool APPEND = false>
__device__ __forceinline__ void run_ring_worker(const DecodeArgs &a, int w, int W, int lane, Seg &seg) {
  if constexpr (APPEND) {  // the fused step's copy of the new rows around the decode work
    AppendCopy<D, 2> copy;
    copy.begin(a, w, lane);
    run_ring_worker<MT, G, D, Seg, false>(a, w, W, lane, seg);
    copy.end(a, w, W, lane);
    return;
  }
  Windows first;
  const Split sp = make_split(count_units<MT>(a, w, W, lane, first), W);
  if (w >= sp.Ws) return;
  if (!seg.start(sp, first, sp.begin(w), sp.begin(w + 1))) return;
  SegInfo cur;
  while (seg.next_segment(cur)) {
    seg.run(cur);
    if (cur.u_lo == 0 && cur.u_hi == cur.n) {
      seg.write_out(cur.s, cur.kvh);
    } else {
      seg.write_partial(cur.first ? 2 * (int64_t)w : 2 * (int64_t)w + 1);
      seg.publish(cur);
    }
  }
  seg.end();
}

// APPEND: the fused step (16-bit caches); BSC: per-block scales (fp8 caches)
template <typename KVT, typename MT, int D, int G, int BS, bool APPEND, bool BSC>
struct SegFor {
  typedef MfmaRegSeg<KVT, MT, D, G, BS, BSC> type;
  __device__ static void run(const DecodeArgs &a, int w, int W, int lane, type &seg) {
    run_worker<MT, G, D>(a, w, W, lane, seg);
  }
};
template <typename MT, int D, int G, int BS, bool APPEND, bool BSC>
struct SegFor<MT, MT, D, G, BS, APPEND, BSC> {
  typedef MfmaRingSeg<MT, D, G, BS, APPEND> type;
  __device__ static void run(const DecodeArgs &a, int w, int W, int lane, type &seg) {
    run_ring_worker<MT, G, D, type, APPEND>(a, w, W, lane, seg);
  }
};

template <typename KVT, typename MT, int D, int G, int BS, bool APPEND, bool BSC = false>
__global__ void __launch_bounds__(64 * kWavesPerWG) decode_mfma(const DecodeArgs a) {
  typedef typename SegFor<KVT, MT, D, G, BS, APPEND, BSC>::type Seg;
  __shared__ __attribute__((aligned(1024))) char lds[kWavesPerWG][Seg::kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  // workgroups are dealt to the 8 XCDs round-robin; number them so that each
  // XCD's workers hold one contiguous stretch of the work order
  const int nb = gridDim.x, b = blockIdx.x;
  const int bx = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  Seg seg(a, lane, lds[wave]);
  SegFor<KVT, MT, D, G, BS, APPEND, BSC>::run(a, bx * kWavesPerWG + wave, nb * kWavesPerWG, lane, seg);
}

template <typename KVT, typename MT, int D, int G>
hipError_t launch_g(const DecodeArgs &a, hipStream_t stream) {
  const dim3 grid(a.num_workers / kWavesPerWG), block(64 * kWavesPerWG);
  if constexpr (__is_same(KVT, MT)) {  // the fused step: 16-bit caches (the ring kernel)
    if (a.append) {
      if (a.block_size == 16)
        hipLaunchKernelGGL((decode_mfma<KVT, MT, D, G, 16, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((decode_mfma<KVT, MT, D, G, 32, true>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if constexpr (!__is_same(KVT, MT)) {  // fp8 with per-block scales: their own variant
    if (a.k_block_scale != nullptr) {
      if (a.block_size == 16)
        hipLaunchKernelGGL((decode_mfma<KVT, MT, D, G, 16, false, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((decode_mfma<KVT, MT, D, G, 32, false, true>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if (a.block_size == 16)
    hipLaunchKernelGGL((decode_mfma<KVT, MT, D, G, 16, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_mfma<KVT, MT, D, G, 32, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <typename KVT, typename MT, int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t stream) {
  switch (a.num_heads / a.num_kv_heads) {
    case 4: return launch_g<KVT, MT, D, 4>(a, stream);
    case 8: return launch_g<KVT, MT, D, 8>(a, stream);
    case 16: return launch_g<KVT, MT, D, 16>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename KVT, typename MT>
hipError_t launch_kv(const DecodeArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return launch_d<KVT, MT, 64>(a, stream);
    case 128: return launch_d<KVT, MT, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_uses_mfma(int kv_kind, int head_dim, int group) {
  return kv_kind != KV_F32 && (head_dim == 64 || head_dim == 128) && (group == 4 || group == 8 || group == 16);
}

int decode_mfma_chunk_tokens() { return CT; }

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream) {
  switch (a.kv_kind) {
    case KV_F16: return launch_kv<f16_t, f16_t>(a, stream);
    case KV_BF16: return launch_kv<bf16_t, bf16_t>(a, stream);
    case KV_FP8:
      if (a.q_kind == KV_F16) return launch_kv<fp8_t, f16_t>(a, stream);
      if (a.q_kind == KV_BF16) return launch_kv<fp8_t, bf16_t>(a, stream);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
