// Paged decode on the vector ALUs: persistent, balanced split-context workers.
//
// The table lookup follows the logical-to-physical translation of the page
// "vLLM框架中的KV cache优化与PagedAttention机制详解" (section 5.1: find the KV range,
// map logical block numbers to physical ones, handle reads that cross blocks;
// section 5.2: translate many block numbers at once, prefetch ahead), with
// the address rule physical = block * block_size + offset of page
// "Paged KVCache：大模型推理显存管理优化方案" (section 2.3).  The per-block score /
// cross-block accumulation split is the one page
// "vLLM推理引擎架构：PagedAttention机制与高吞吐推理" (section 2.3) describes.
//
// Work distribution is in pa_sched.h: every wavefront is one worker that
// streams an equal share of all (sequence, kv head) contexts.
//
// Data movement (the whole cost of this kernel): a token's K row for one kv
// head is head_dim * elem bytes, contiguous.  LPR lanes cover it with 16-byte
// loads, so one wave-wide load reads TPW = 64 / LPR consecutive tokens of one
// block.  A chunk is NL such loads (CH = TPW * NL tokens) of K and the same of
// V.  The loop is a rolling pipeline: the next chunk's K loads are issued as
// soon as this chunk's scores are computed, its V loads as soon as this
// chunk's V rows are accumulated, so a wave always has a chunk's worth of K or
// V in flight.  Block-table entries come through the scalar unit one chunk
// ahead.  Loads past the end of a segment are redirected to its last token
// (already in cache), never to another worker's tokens.
//
// Arithmetic (fp32): score = (q . K) * scale * log2(e), the dot product per lane
// with v_dot2 (16-bit and fp8 KV, fp8 converted exactly to the query's type)
// or FMAs (fp32 KV), then a DPP sum over the LPR
// lanes of a token; a running reference max m and sum l, rescaled by
// exp2(m_old - m_new) only when a chunk's max exceeds m by more than 8 (so
// weights stay below 2^8 and most chunks skip the rescale); acc += p * V.  Masked tokens get p = 0 and a
// finite (duplicated) V row, so nothing poisons the sum.
#include "pa_sched.h"

namespace pa {

namespace {

constexpr int kWavesPerWG = 4;
constexpr float kSlack = 8.0f;  // how far (log2 units) scores may exceed the running reference max

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

// Block tables and context lengths are never written during a launch: reading
// them through the constant address space lets uniform reads use the scalar unit.
typedef const __attribute__((address_space(4))) int32_t const_i32;

__device__ __forceinline__ const_i32 *as_const(const int32_t *p) { return (const_i32 *)(uintptr_t)p; }

// One lane's slice of a query row and its dot product with a 16-byte K slice.
template <typename KVT, typename QT> struct QSlice;

template <> struct QSlice<f16_t, f16_t> {
  u32x4 w;
  __device__ void load(const void *q, int64_t off) { w = ld16(reinterpret_cast<const _Float16 *>(q) + off); }
  __device__ float dot(u32x4 k) const {
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qa = w[i], ka = k[i];
      d = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, qa), __builtin_bit_cast(h2_t, ka), d, false);
    }
    return d;
  }
};

template <> struct QSlice<bf16_t, bf16_t> {
  u32x4 w;
  __device__ void load(const void *q, int64_t off) { w = ld16(reinterpret_cast<const uint16_t *>(q) + off); }
  __device__ float dot(u32x4 k) const {
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qa = w[i], ka = k[i];
      d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, qa), __builtin_bit_cast(b2_t, ka), d, false);
    }
    return d;
  }
};

template <> struct QSlice<f32_t, f32_t> {
  float f[4];
  __device__ void load(const void *q, int64_t off) { Elem<f32_t>::unpack(ld16(reinterpret_cast<const float *>(q) + off), f); }
  __device__ float dot(u32x4 k) const {
    float kf[4];
    Elem<f32_t>::unpack(k, kf);
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) d = __builtin_fmaf(f[i], kf[i], d);
    return d;
  }
};

// fp8 K with a 16-bit query: 16 codes per slice, converted exactly to the
// query's type in pairs, then v_dot2 against the packed query slice
template <typename QT> struct QSliceFp8 {
  u32x4 w[2];  // 16 query elements
  __device__ void load(const void *q, int64_t off) {
    const char *p = reinterpret_cast<const char *>(q) + off * 2;
    w[0] = ld16(p);
    w[1] = ld16(p + 16);
  }
  __device__ float dot(u32x4 k) const {
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // codes 4i .. 4i+3 against query elements 4i .. 4i+3
      const uint32_t k01 = __is_same(QT, f16_t) ? fp8x2_to_f16x2<false>(k[i]) : fp8x2_to_bf16x2<false>(k[i]);
      const uint32_t k23 = __is_same(QT, f16_t) ? fp8x2_to_f16x2<true>(k[i]) : fp8x2_to_bf16x2<true>(k[i]);
      const uint32_t q01 = w[i >> 1][2 * (i & 1)], q23 = w[i >> 1][2 * (i & 1) + 1];
      if constexpr (__is_same(QT, f16_t)) {
        d = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, q01), __builtin_bit_cast(h2_t, k01), d, false);
        d = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, q23), __builtin_bit_cast(h2_t, k23), d, false);
      } else {
        d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, q01), __builtin_bit_cast(b2_t, k01), d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, q23), __builtin_bit_cast(b2_t, k23), d, false);
      }
    }
    return d;
  }
};
template <> struct QSlice<fp8_t, f16_t> : QSliceFp8<f16_t> {};
template <> struct QSlice<fp8_t, bf16_t> : QSliceFp8<bf16_t> {};

// VEC consecutive output values of one lane, rounded to the output dtype.
template <typename OT, int VEC>
__device__ __forceinline__ void store_vec(void *base, int64_t off, const float *x) {
  if constexpr (sizeof(typename OT::storage) == 4) {
#pragma unroll
    for (int j = 0; j < VEC; j += 4) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(uint32_t, x[j + i]);
      st16(reinterpret_cast<float *>(base) + off + j, w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < VEC; j += 8) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo, hi;
        if constexpr (__is_same(OT, f16_t)) {
          lo = __builtin_bit_cast(uint16_t, (_Float16)x[j + 2 * i]);
          hi = __builtin_bit_cast(uint16_t, (_Float16)x[j + 2 * i + 1]);
        } else {
          lo = f32_to_bf16_rne(x[j + 2 * i]);
          hi = f32_to_bf16_rne(x[j + 2 * i + 1]);
        }
        w[i] = lo | (hi << 16);
      }
      st16(reinterpret_cast<uint16_t *>(base) + off + j, w);
    }
  }
}

// BSC: fp8 caches with one scale per (block, kv head) (a variant of its own,
// so that the other launches carry none of its work)
template <typename KVT, typename QT, int D, int G, int BS, int NL, bool APPEND = false, bool BSC = false>
struct ValuSeg {
  static constexpr int VEC = Elem<KVT>::kPer16;  // KV elements per 16-byte load
  static constexpr int LPR = D / VEC;            // lanes per token row
  static constexpr int TPW = 64 / LPR;           // tokens per wave-wide load
  static constexpr int CH = TPW * NL;            // tokens per chunk
  static constexpr int LOG2BS = BS == 16 ? 4 : 5;
  static constexpr int EB = Elem<KVT>::kBytes;
  static_assert(LPR >= 4 && LPR <= 32, "a row must span 4..32 lanes");
  static_assert(BS % TPW == 0, "a wave-wide load must stay inside one block");

  const DecodeArgs &a;
  const int lane, r, tg;  // lane, 16-byte slice of the row, token of a wave-wide load
  float m[G], l[G], acc[G][VEC];
  float vsc;              // the segment's output scale (fp8 value scale)

  __device__ ValuSeg(const DecodeArgs &args, int ln) : a(args), lane(ln), r(ln % LPR), tg(ln / LPR) {}

  // Block ids of the chunk starting at cs: the chunk spans NBC blocks (one
  // when it is shorter than a block), and wave-wide load i reads block
  // (i * TPW) / BS of them.  A load past `last` reads last's block, which is
  // always one of the chunk's own.
  static constexpr int NBC = CH >= BS ? CH / BS : 1;
  __device__ __forceinline__ void fetch_blocks(const_i32 *bt, int cs, int last, int *blk) const {
    int e[NBC];
#pragma unroll
    for (int j = 0; j < NBC; ++j) e[j] = bt[min(cs + j * BS, last) >> LOG2BS];
#pragma unroll
    for (int j = 0; j < NBC; ++j) e[j] = e[j] < 0 ? 0 : (e[j] >= a.num_blocks ? a.num_blocks - 1 : e[j]);
#pragma unroll
    for (int i = 0; i < NL; ++i) blk[i] = e[NBC == 1 ? 0 : (i * TPW) / BS];
  }

  // the block's base address is uniform (scalar registers); each lane adds a
  // 32-bit offset inside the block
  __device__ __forceinline__ void issue(const char *base, int64_t sb, int64_t st, int cs, int last, const int *blk,
                                        u32x4 *dst) const {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int t = min(cs + i * TPW + tg, last);
      const char *bb = base + (int64_t)blk[i] * sb * EB;
      const char *pl = bb + (uint32_t)(((t & (BS - 1)) * (uint32_t)st + r * VEC) * EB);
      dst[i] = ld16_stream(pl);
    }
  }

  // A fused step (APPEND) whose new token goes to a slot of the pool (the
  // slot this launch writes): the token stays out of the paged range of its
  // item's last segment, and opens the item's first segment instead, its K
  // and V rows read from k_new / v_new.  The softmax over the item is the
  // same set of scores; only the order of the sums changes.
  __device__ __forceinline__ int paged_end(const SegInfo &g) const {
    return g.t_hi - (APPEND && g.u_hi == g.n && append_writes(a, g.s) ? 1 : 0);
  }
  __device__ __forceinline__ void load_new(const SegInfo &g, u32x4 &kd, u32x4 &vd) const {
    const int64_t c = r * VEC;
    kd = ld16(reinterpret_cast<const char *>(a.k_new) + ((int64_t)g.s * a.kn_ss + (int64_t)g.kvh * a.kn_sh + c) * EB);
    vd = ld16(reinterpret_cast<const char *>(a.v_new) + ((int64_t)g.s * a.vn_ss + (int64_t)g.kvh * a.vn_sh + c) * EB);
  }
  // the running state after the new token alone: its score is the reference
  // maximum (the same on every lane: each lane group holds the whole row), and
  // token group 0 holds its weight 1 and its value row
  __device__ __forceinline__ void open_with_new(float qk) {
    float sn[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sn[h] = q[h].dot(kn);
    group_sum_n<LPR, G>(sn);
    float vf[VEC];
    Elem<KVT>::unpack(vn, vf);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = sn[h] * qk;
      l[h] = tg == 0 ? 1.0f : 0.0f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[h][v] = tg == 0 ? vf[v] : 0.0f;
    }
  }

  // where a segment's rows live
  struct Ptrs {
    const_i32 *bt;
    const char *kb, *vb;
    int last;  // the last token of the paged range (loads past it read it again)
    const float *ksb, *vsb;  // fp8 per-block scales: this layer's and kv head's (stride num_kv_heads per block), or null
  };
  __device__ __forceinline__ Ptrs ptrs(const SegInfo &g) const {
    Ptrs p;
    p.bt = as_const(a.block_tables) + (int64_t)seq_of(a, g.s) * a.bt_ss;
    p.kb = reinterpret_cast<const char *>(a.k_cache) + (k_layer(a, g.s) + (int64_t)g.kvh * a.k_sh) * EB;  // uniform
    p.vb = reinterpret_cast<const char *>(a.v_cache) + (v_layer(a, g.s) + (int64_t)g.kvh * a.v_sh) * EB;
    // a fused step's segment that holds only the new token has an empty paged
    // range: the loads issued ahead for it read the token before (for a
    // sequence of one token, position 0), in bounds, and are never used
    p.last = APPEND ? max(paged_end(g) - 1, 0) : g.t_hi - 1;
    p.ksb = p.vsb = nullptr;
    if (BSC) {
      const int64_t o = (int64_t)layer_of(a, g.s) * a.num_blocks * a.num_kv_heads + g.kvh;
      p.ksb = a.k_block_scale + o;
      p.vsb = a.v_block_scale + o;
    }
    return p;
  }

  // fp8 caches with per-block scales: the key and value scales of the
  // blocks that load i of a chunk reads (scalar loads, a chunk ahead of their
  // use)
  static_assert(!BSC || __is_same(KVT, fp8_t), "per-block scales are for fp8 caches");
  __device__ __forceinline__ void fetch_scales(const float *ksb, const float *vsb, const int *blk, float *ks,
                                               float *vs) const {
    typedef const __attribute__((address_space(4))) float cf;
#pragma unroll
    for (int i = 0; i < NL; ++i) ks[i] = vs[i] = 1.0f;
    if (!BSC) return;
#pragma unroll
    for (int j = 0; j < NBC; ++j) {
      const int i0 = NBC == 1 ? 0 : (j * BS) / TPW;  // the first load in block j of the chunk
      const int64_t off = (int64_t)blk[i0] * a.num_kv_heads;
      const float kx = ((cf *)(uintptr_t)ksb)[off], vx = ((cf *)(uintptr_t)vsb)[off];
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if ((NBC == 1 ? 0 : (i * TPW) / BS) == j) {
          ks[i] = kx;
          vs[i] = vx;
        }
    }
  }
  __device__ __forceinline__ void load_q(const SegInfo &g, QSlice<KVT, QT> *dst) const {
    const int64_t qr = q_row(a, g.s);
#pragma unroll
    for (int h = 0; h < G; ++h) dst[h].load(a.q, qr + (int64_t)(g.kvh * G + h) * a.q_sh + r * VEC);
  }

  // pipeline state carried from one segment into the next
  QSlice<KVT, QT> q[G];
  int blk[NL];
  float kbs[NL], vbs[NL];  // the current chunk's per-load block scales (fp8 with per-block scales; else 1)
  u32x4 kr[NL], vr[NL];
  u32x4 kn, vn;  // fused step: the new token's K and V row slices of the current segment's item

  // q, block ids and the K / V loads of g's first chunk; K before V, so that
  // the first wait of the chunk loop is for K alone
  __device__ void begin(const SegInfo &g, const Walker &) { begin(g); }
  __device__ void publish(const SegInfo &g, const Split &sp) {
    finish_partial<QT, G, D>(a, g.s, g.kvh, g.a0, g.n, sp, lane);
  }
  __device__ void end() {}

  __device__ void begin(const SegInfo &g) {
    const Ptrs p = ptrs(g);
    load_q(g, q);
    if constexpr (APPEND) load_new(g, kn, vn);
    fetch_blocks(p.bt, g.t_lo, p.last, blk);
    if constexpr (BSC) fetch_scales(p.ksb, p.vsb, blk, kbs, vbs);
    __builtin_amdgcn_sched_barrier(0);
    issue(p.kb, a.k_sb, a.k_st, g.t_lo, p.last, blk, kr);
    __builtin_amdgcn_sched_barrier(0);
    issue(p.vb, a.v_sb, a.v_st, g.t_lo, p.last, blk, vr);
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ void run(const SegInfo &g, const SegInfo &nx, bool has) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.0f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[h][v] = 0.0f;
    }
    const ItemScale isc = seg_scale<KVT>(a, g.s, g.kvh);
    vsc = isc.v;
    if constexpr (APPEND) {
      if (g.u_lo == 0 && append_writes(a, g.s)) open_with_new(isc.qk);
    }
    const int pend = APPEND ? paged_end(g) : g.t_hi;
    // empty: a fused step's segment holding only the new token (its state is
    // complete in token group 0), or context_lens changed under the launch
    if (pend <= g.t_lo) {
      if (has) begin(nx);
      return;
    }
    const Ptrs p = ptrs(g);
    // the chunk after this segment's last one: the next segment's first (or,
    // for the range's last segment, this last chunk again -- a cache hit, unused)
    const Ptrs pn = has ? ptrs(nx) : p;
    QSlice<KVT, QT> qn[G];
    load_q(has ? nx : g, qn);
    u32x4 knn, vnn;
    if constexpr (APPEND) load_new(has ? nx : g, knn, vnn);

    const int nch = (pend - g.t_lo + CH - 1) / CH;
    int cs = g.t_lo;
    for (int c = 0; c < nch; ++c) {
      const bool lastc = c + 1 == nch;
      const int cn = lastc ? (has ? nx.t_lo : cs) : cs + CH;
      const_i32 *btn = lastc ? pn.bt : p.bt;
      const char *kbn = lastc ? pn.kb : p.kb;
      const char *vbn = lastc ? pn.vb : p.vb;
      const int lastn = lastc ? pn.last : p.last;
      int nblk[NL];
      fetch_blocks(btn, cn, lastn, nblk);
      float nkbs[NL], nvbs[NL];
      if constexpr (BSC) fetch_scales(lastc ? pn.ksb : p.ksb, lastc ? pn.vsb : p.vsb, nblk, nkbs, nvbs);
      // the scheduler would otherwise sink table reads and loads down to their
      // uses and drain the pipeline: keep the program order at these points
      __builtin_amdgcn_sched_barrier(0);

      float sc[G][NL];
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h][i] = q[h].dot(kr[i]);
      group_sum_n<LPR, G * NL>(&sc[0][0]);
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const bool valid = cs + i * TPW + tg <= p.last;
#pragma unroll
        for (int h = 0; h < G; ++h) sc[h][i] = valid ? sc[h][i] * (BSC ? isc.qk * kbs[i] : isc.qk) : -INFINITY;
      }
      __builtin_amdgcn_sched_barrier(0);
      issue(kbn, a.k_sb, a.k_st, cn, lastn, nblk, kr);
      __builtin_amdgcn_sched_barrier(0);

#pragma unroll
      for (int h = 0; h < G; ++h) {
        float cm = sc[h][0];
#pragma unroll
        for (int i = 1; i < NL; ++i) cm = fmaxf(cm, sc[h][i]);
        cm = across_groups_max<LPR>(cm);
        // lazy rescale: the reference max moves only when a score exceeds it by
        // more than kSlack (log2 units); weights stay below 2^kSlack
        if (cm > m[h] + kSlack) {  // uniform: m and cm are the same on every lane
          const float mn = fmaxf(m[h], cm);
          const float alpha = fast_exp2(m[h] - mn);
          l[h] *= alpha;
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[h][v] *= alpha;
          m[h] = mn;
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) sc[h][i] = fast_exp2(sc[h][i] - m[h]);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float vf[VEC];
        Elem<KVT>::unpack(vr[i], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          l[h] += sc[h][i];
          const float w = BSC ? sc[h][i] * vbs[i] : sc[h][i];  // the weight times its block's value scale
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[h][v] = __builtin_fmaf(w, vf[v], acc[h][v]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      issue(vbn, a.v_sb, a.v_st, cn, lastn, nblk, vr);
      __builtin_amdgcn_sched_barrier(0);
      cs = cn;
#pragma unroll
      for (int i = 0; i < NL; ++i) blk[i] = nblk[i];
      if constexpr (BSC) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          kbs[i] = nkbs[i];
          vbs[i] = nvbs[i];
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) q[h] = qn[h];
    if constexpr (APPEND) {
      kn = knn;
      vn = vnn;
    }

    // every lane ends with the totals of its row slice over all tokens of the segment
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] = across_groups_sum<LPR>(l[h]);
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[h][v] = across_groups_sum<LPR>(acc[h][v]);
    }
  }

  __device__ void write_out(int s, int kvh) const {
    if (tg != 0) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float o[VEC];
      const float inv = vsc / l[h];
#pragma unroll
      for (int v = 0; v < VEC; ++v) o[v] = acc[h][v] * inv;
      const int64_t off = o_row(a, s) + (int64_t)(kvh * G + h) * a.o_sh + r * VEC;
      if (a.out_f32)
        store_vec<f32_t, VEC>(a.out, off, o);
      else
        store_vec<QT, VEC>(a.out, off, o);
    }
  }

  __device__ void write_partial(int64_t slot) const {
    if (tg == 0) {
      const int64_t pacc = slot_acc<G, D>(slot);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int v = 0; v < VEC; v += 4) store_shared4(a, pacc + h * D + r * VEC + v, &acc[h][v]);
    }
    if (lane == 0) {
      const int64_t pml = slot_ml<G>(slot);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        store_shared_ml(a, pml + 2 * h, m[h]);
        store_shared_ml(a, pml + 2 * h + 1, l[h]);
      }
    }
  }
};

template <typename KVT, typename QT, int D, int G, int BS, int NL, bool APPEND, bool BSC = false>
__global__ void __launch_bounds__(64 * kWavesPerWG) decode_valu(const DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  // workgroups are dealt to the 8 XCDs round-robin; number them so that each
  // XCD's workers hold one contiguous stretch of the work order
  const int nb = gridDim.x, b = blockIdx.x;
  const int bx = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  ValuSeg<KVT, QT, D, G, BS, NL, APPEND, BSC> seg(a, lane);
  run_worker<QT, G, D, ValuSeg<KVT, QT, D, G, BS, NL, APPEND, BSC>, APPEND ? Elem<KVT>::kBytes : 0>(
      a, bx * kWavesPerWG + wave, nb * kWavesPerWG, lane, seg);
}

// loads per chunk: fewer for larger groups, whose query, score and accumulator
// registers grow with G
template <int G> constexpr int nl_for() { return G == 1 ? 8 : (G == 2 ? 4 : (G == 4 ? 2 : 1)); }

template <typename KVT, typename QT, int D, int G>
hipError_t launch_one(const DecodeArgs &a, hipStream_t stream) {
  constexpr int NL = nl_for<G>();
  const dim3 grid(a.num_workers / kWavesPerWG), block(64 * kWavesPerWG);
  if constexpr (!__is_same(KVT, fp8_t)) {  // the fused step copies rows of the cache's own dtype
    if (a.append) {
      if (a.block_size == 16)
        hipLaunchKernelGGL((decode_valu<KVT, QT, D, G, 16, NL, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((decode_valu<KVT, QT, D, G, 32, NL, true>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if constexpr (__is_same(KVT, fp8_t)) {  // per-block scales: their own variant
    if (a.k_block_scale != nullptr) {
      if (a.block_size == 16)
        hipLaunchKernelGGL((decode_valu<KVT, QT, D, G, 16, NL, false, true>), grid, block, 0, stream, a);
      else
        hipLaunchKernelGGL((decode_valu<KVT, QT, D, G, 32, NL, false, true>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  }
  if (a.block_size == 16)
    hipLaunchKernelGGL((decode_valu<KVT, QT, D, G, 16, NL, false>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_valu<KVT, QT, D, G, 32, NL, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// groups of 4 and more go to the matrix cores, except for fp32 caches
template <typename KVT, typename QT, int D>
hipError_t dispatch_group(const DecodeArgs &a, hipStream_t stream) {
  switch (a.num_heads / a.num_kv_heads) {
    case 1: return launch_one<KVT, QT, D, 1>(a, stream);
    case 2: return launch_one<KVT, QT, D, 2>(a, stream);
  }
  if constexpr (__is_same(KVT, f32_t)) {
    switch (a.num_heads / a.num_kv_heads) {
      case 4: return launch_one<KVT, QT, D, 4>(a, stream);
      case 8: return launch_one<KVT, QT, D, 8>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

template <typename KVT, typename QT>
hipError_t dispatch_dim(const DecodeArgs &a, hipStream_t stream) {
  switch (a.head_dim) {
    case 64: return dispatch_group<KVT, QT, 64>(a, stream);
    case 128: return dispatch_group<KVT, QT, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int decode_chunk_tokens(int kv_kind, int head_dim, int group) {
  if (decode_uses_mfma(kv_kind, head_dim, group)) return decode_mfma_chunk_tokens();
  const int vec = kv_kind == KV_F32 ? 4 : (kv_kind == KV_FP8 ? 16 : 8);
  const int tpw = 64 / (head_dim / vec);
  const int nl = group == 1 ? 8 : (group == 2 ? 4 : (group == 4 ? 2 : 1));
  return tpw * nl;
}

bool decode_supported(int kv_kind, int q_kind, int head_dim, int group) {
  const bool pair = (kv_kind == q_kind && kv_kind != KV_FP8) ||
                    (kv_kind == KV_FP8 && (q_kind == KV_F16 || q_kind == KV_BF16));
  if (!pair || (head_dim != 64 && head_dim != 128)) return false;
  if (group == 1 || group == 2) return true;
  if (kv_kind == KV_F32) return group == 4 || group == 8;
  return decode_uses_mfma(kv_kind, head_dim, group);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (decode_uses_mfma(a.kv_kind, a.head_dim, a.num_heads / a.num_kv_heads)) return launch_decode_mfma(a, stream);
  switch (a.kv_kind) {
    case KV_F32: return dispatch_dim<f32_t, f32_t>(a, stream);
    case KV_F16: return dispatch_dim<f16_t, f16_t>(a, stream);
    case KV_BF16: return dispatch_dim<bf16_t, bf16_t>(a, stream);
    case KV_FP8:
      if (a.q_kind == KV_F16) return dispatch_dim<fp8_t, f16_t>(a, stream);
      if (a.q_kind == KV_BF16) return dispatch_dim<fp8_t, bf16_t>(a, stream);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
