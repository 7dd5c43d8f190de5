// Host sanitizer run of the C ABI's host side: pa_api.cpp and pa_validate.cpp
// are compiled together with this driver under AddressSanitizer and
// UndefinedBehaviorSanitizer (the kernels' objects are linked as built, their
// host parts uninstrumented), and the argument checks of every entry point
// and the index checks of PA_FLAG_VALIDATE run on bad and good inputs.  Every
// ABI call here fails before anything is enqueued (fake device pointers are
// never dereferenced: no GPU is used), so this runs on any host.  Any
// out-of-bounds access, use after free or undefined operation ends the run
// with a report; the status checks pin the paths taken.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>
#include <vector>

#include "pa.h"
#include "pa_validate.h"

static int fails = 0;
#define EXPECT(c)                                                      \
  do {                                                                 \
    if (!(c)) {                                                        \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++fails;                                                         \
    }                                                                  \
  } while (0)

namespace {

void *const kFake = reinterpret_cast<void *>(uintptr_t(0x7F0000000000));  // never dereferenced

pa_tensor T(std::initializer_list<int64_t> shape, int dtype, void *data = kFake) {
  pa_tensor t;
  std::memset(&t, 0, sizeof t);
  t.data = data;
  t.dtype = dtype;
  t.ndim = (int32_t)shape.size();
  int i = 0;
  for (int64_t n : shape) t.shape[i++] = n;
  int64_t acc = 1;
  for (int k = t.ndim - 1; k >= 0; --k) {
    t.stride[k] = acc;
    acc *= t.shape[k];
  }
  return t;
}

pa_opts Opts(bool workspace = true) {
  pa_opts o;
  std::memset(&o, 0, sizeof o);
  o.num_workers = 64;  // no device query for the default
  if (workspace) {
    o.workspace = kFake;
    o.workspace_bytes = size_t(1) << 40;
  }
  return o;
}

// an error status and a message naming something
#define expect_error(...) expect_error_at(__LINE__, __VA_ARGS__)
void expect_error_at(int line, pa_status s, pa_status want = PA_OK) {
  const char *m = pa_last_error();
  if (s == PA_OK || (want != PA_OK && s != want) || !m || !*m) {
    std::fprintf(stderr, "FAIL line %d: status %d (want %d): %s\n", line, (int)s, (int)want, m ? m : "(null)");
    ++fails;
  }
}

struct Decode {
  pa_tensor out, q, k, v, bt, cl;
  int32_t bs = 16, hkv = 2;
  float scale = 0.088f;
  Decode(int64_t S = 4, int64_t H = 8, int64_t Hkv = 2, int64_t D = 128, int64_t NB = 64, int64_t W = 8,
         int kv = PA_F16, int qd = PA_F16)
      : out(T({S, H, D}, qd)), q(T({S, H, D}, qd)), k(T({NB, 16, Hkv, D}, kv)), v(T({NB, 16, Hkv, D}, kv)),
        bt(T({S, W}, PA_I32)), cl(T({S}, PA_I32)), hkv((int32_t)Hkv) {}
  pa_status run(const pa_opts &o) const { return pa_decode(out, q, k, v, bt, cl, bs, scale, hkv, &o); }
};

void abi_argument_checks() {
  for (int s = 1; s >= -12; --s) EXPECT(pa_status_string((pa_status)s) && *pa_status_string((pa_status)s));
  EXPECT(pa_version() && *pa_version());
  EXPECT(pa_decode_workspace_size(4, 8, 2, 128, 64) > 0);
  EXPECT(pa_decode_workspace_size(4, 8, 3, 128, 64) == 0);
  EXPECT(pa_decode_workspace_size(-1, 8, 2, 128, 64) == 0);
  EXPECT(pa_decode_num_workers(5) == 8);
  EXPECT(pa_prefill_workspace_size() > 0);
  EXPECT(pa_decode_static_scratch_bytes() > 0);

  {  // decode: each argument broken in turn
    Decode a;
    Decode b = a;
    b.q.data = nullptr;
    expect_error(b.run(Opts()), PA_ERR_NULL);
    b = a;
    b.k.dtype = PA_BF16;
    expect_error(b.run(Opts()), PA_ERR_DTYPE);
    b = a;
    b.bt.dtype = PA_I64;
    expect_error(b.run(Opts()), PA_ERR_DTYPE);
    b = a;
    b.q.shape[2] = 64;
    expect_error(b.run(Opts()));
    b = a;
    b.k.ndim = 7;  // past the five dimensions a tensor holds
    expect_error(b.run(Opts()));
    b = a;
    b.k.stride[0] = -b.k.stride[0];
    expect_error(b.run(Opts()));
    b = a;
    b.k.stride[1] = std::numeric_limits<int64_t>::max() / 2;
    expect_error(b.run(Opts()));
    b = a;
    b.bt.shape[0] = std::numeric_limits<int64_t>::max();
    expect_error(b.run(Opts()));
    b = a;
    b.hkv = 3;
    expect_error(b.run(Opts()));
    b = a;
    b.hkv = 0;
    expect_error(b.run(Opts()));
    b = a;
    b.scale = std::nanf("");
    expect_error(b.run(Opts()), PA_ERR_ARG);
    b = a;
    b.bs = 7;
    expect_error(b.run(Opts()));
    pa_opts o = Opts();
    o.partition_size = 24;
    expect_error(a.run(o), PA_ERR_ARG);
    o = Opts();
    o.flags = 2;
    expect_error(a.run(o), PA_ERR_ARG);
    o = Opts();
    o.num_workers = -4;
    expect_error(a.run(o), PA_ERR_ARG);
    o = Opts(false);
    expect_error(a.run(o), PA_ERR_WORKSPACE);
    o = Opts();
    o.workspace_bytes = 100;
    expect_error(a.run(o), PA_ERR_WORKSPACE);
    o = Opts();
    o.k_head_scales = reinterpret_cast<const float *>(kFake);  // without v_head_scales
    expect_error(a.run(o));
    Decode f(4, 8, 2, 128, 64, 8, PA_FP8_E4M3, PA_F32);
    expect_error(f.run(Opts()), PA_ERR_DTYPE);
    // the validated call refuses fake pointers (nothing to copy from) before any launch
    o = Opts();
    o.flags = PA_FLAG_VALIDATE;
    expect_error(a.run(o));
    // the static entry point refuses a caller workspace, and a request past its scratch
    expect_error(pa_decode_static(a.out, a.q, a.k, a.v, a.bt, a.cl, a.bs, a.scale, a.hkv, &o), PA_ERR_ARG);
    Decode big(1 << 30, 8, 2, 128, 64, 8);
    pa_opts so = Opts(false);
    expect_error(pa_decode_static(big.out, big.q, big.k, big.v, big.bt, big.cl, big.bs, big.scale, big.hkv, &so),
                 PA_ERR_WORKSPACE);
    // the fused step: new rows of the wrong shape, fp8 caches refused
    pa_tensor kn = T({4, 2, 128}, PA_F16), vn = T({4, 2, 128}, PA_F16), sm = T({4}, PA_I64);
    pa_tensor kn_bad = T({4, 2, 64}, PA_F16);
    expect_error(pa_decode_append(a.out, a.q, kn_bad, vn, a.k, a.v, sm, a.bt, a.cl, a.bs, a.scale, a.hkv, &o));
    o = Opts();
    expect_error(pa_decode_append(f.out, f.q, kn, vn, f.k, f.v, sm, f.bt, f.cl, f.bs, f.scale, f.hkv, &o));
    // several layers: caches of rank 5 with mismatched layer counts
    pa_tensor lo = T({3, 4, 8, 128}, PA_F16), lq = T({3, 4, 8, 128}, PA_F16);
    pa_tensor lk = T({2, 64, 16, 2, 128}, PA_F16), lv = T({3, 64, 16, 2, 128}, PA_F16);
    expect_error(pa_decode_layers(lo, lq, lk, lv, a.bt, a.cl, a.bs, a.scale, a.hkv, &o), PA_ERR_SHAPE);
  }
  {  // prefill
    pa_tensor out = T({40, 8, 128}, PA_F16), q = T({40, 8, 128}, PA_F16), k = T({64, 16, 2, 128}, PA_F16);
    pa_tensor bt = T({4, 8}, PA_I32), cl = T({4}, PA_I32), qsl = T({5}, PA_I32), qsl_bad = T({4}, PA_I32);
    pa_opts o = Opts(false);
    expect_error(pa_prefill(out, q, k, k, bt, cl, qsl_bad, 16, 0.088f, 2, &o));
    expect_error(pa_prefill(out, q, k, k, bt, cl, qsl, 16, 0.0f, 2, &o), PA_ERR_ARG);
    pa_tensor qn = q;
    qn.data = nullptr;
    expect_error(pa_prefill(out, qn, k, k, bt, cl, qsl, 16, 0.088f, 2, &o), PA_ERR_NULL);
    o.flags = 4;
    expect_error(pa_prefill(out, q, k, k, bt, cl, qsl, 16, 0.088f, 2, &o), PA_ERR_ARG);
  }
  {  // cache write and block copies
    pa_tensor kn = T({6, 2, 128}, PA_F16), kc = T({64, 16, 2, 128}, PA_F16), sm = T({6}, PA_I64);
    pa_tensor sm_bad = T({5}, PA_I64), kc8 = T({64, 16, 2, 128}, PA_FP8_E4M3);
    pa_opts o = Opts(false);
    expect_error(pa_cache_write(kn, kn, kc, kc, sm_bad, &o));
    expect_error(pa_cache_write(kn, kn, kc8, kc8, T({6}, PA_F32), &o));
    o.k_scale = -1.0f;
    expect_error(pa_cache_write(kn, kn, kc8, kc8, sm, &o));
    o = Opts(false);
    pa_tensor map = T({3, 2}, PA_I64), map_bad = T({3, 3}, PA_I64), other = T({65, 16, 2, 128}, PA_F16);
    expect_error(pa_copy_blocks(kc, kc, kc, kc, map_bad, &o));
    expect_error(pa_copy_blocks(kc, kc, other, other, map, &o));
    expect_error(pa_copy_blocks(kc, kc, kc, kc, map, &o));  // fake pointers: refused, nothing copied
  }
  {  // the streaming-read probe
    pa_opts o = Opts(false);
    uint32_t *parts = static_cast<uint32_t *>(kFake);
    const char *misaligned = static_cast<const char *>(kFake) + 4;
    expect_error(pa_stream_read(nullptr, 1024, 4, 4, 1, parts, &o), PA_ERR_NULL);
    expect_error(pa_stream_read(kFake, 1000, 4, 4, 1, parts, &o), PA_ERR_SHAPE);
    expect_error(pa_stream_read(kFake, 0, 4, 4, 1, parts, &o), PA_ERR_SHAPE);
    expect_error(pa_stream_read(misaligned, 1024, 4, 4, 1, parts, &o), PA_ERR_LAYOUT);
    expect_error(pa_stream_read(kFake, 1024, 0, 4, 1, parts, &o), PA_ERR_ARG);
    expect_error(pa_stream_read(kFake, 1024, 65537, 4, 1, parts, &o), PA_ERR_ARG);
    expect_error(pa_stream_read(kFake, 1024, 4, 3, 1, parts, &o), PA_ERR_UNSUPPORTED);
    o.flags = 1;  // PA_FLAG_VALIDATE: nothing to check here
    expect_error(pa_stream_read(kFake, 1024, 4, 4, 1, parts, &o), PA_ERR_ARG);
    o = Opts(false);
    expect_error(pa_stream_read(kFake, 1024, 4, 4, 1, parts, &o), PA_ERR_ARG);  // fake pointer: refused
  }
}

pa::HostInts H(int64_t rows, int64_t cols, std::vector<int64_t> v) {
  pa::HostInts h;
  h.rows = rows;
  h.cols = cols;
  h.v = std::move(v);
  return h;
}

void contains(const char *needle) {
  const char *m = pa_last_error();
  EXPECT(m && std::strstr(m, needle));
  if (!(m && std::strstr(m, needle))) std::fprintf(stderr, "  message: %s\n", m ? m : "(null)");
}

void validation_checks() {
  // tables: 3 sequences, 4 blocks of 16 per row, a pool of 10 blocks
  pa::HostInts bt = H(3, 4, {0, 1, 2, 3, 4, 5, 99, 99, 6, 7, 8, 9});
  pa::HostInts cl = H(3, 1, {64, 32, 0});
  EXPECT(pa::check_tables(bt, cl, 16, 10) == PA_OK);  // entries past a context are never read
  pa::HostInts cl_long = H(3, 1, {65, 32, 0});
  EXPECT(pa::check_tables(bt, cl_long, 16, 10) == PA_ERR_BAD_INDEX);
  contains("context_lens[0]");
  pa::HostInts cl_neg = H(3, 1, {64, -1, 0});
  EXPECT(pa::check_tables(bt, cl_neg, 16, 10) == PA_ERR_BAD_INDEX);
  pa::HostInts cl_more = H(3, 1, {64, 33, 0});  // now block_tables[1][2] = 99 is read
  EXPECT(pa::check_tables(bt, cl_more, 16, 10) == PA_ERR_BAD_INDEX);
  contains("block_tables[1][2]");
  pa::HostInts bt_neg = H(3, 4, {0, 1, 2, -3, 4, 5, 99, 99, 6, 7, 8, 9});
  EXPECT(pa::check_tables(bt_neg, cl, 16, 10) == PA_ERR_BAD_INDEX);

  // a fused step's slots: position L - 1 of each sequence, distinct
  pa::HostInts slots = H(3, 1, {3 * 16 + 15, 5 * 16 + 15, -1});
  EXPECT(pa::check_new_token_slots(slots, bt, cl, 16, 160) == PA_OK);
  pa::HostInts slots_off = H(3, 1, {3 * 16 + 14, 5 * 16 + 15, -1});
  EXPECT(pa::check_new_token_slots(slots_off, bt, cl, 16, 160) == PA_ERR_BAD_INDEX);
  contains("slot_mapping[0]");
  pa::HostInts slots_skip = H(3, 1, {-1, 1000, 7});  // skipped (< 0, past the pool, empty context)
  EXPECT(pa::check_new_token_slots(slots_skip, bt, cl, 16, 160) == PA_OK);

  // a cache write's slots
  EXPECT(pa::check_distinct_slots(H(4, 1, {5, 9, -1, 1000}), 160) == PA_OK);
  EXPECT(pa::check_distinct_slots(H(4, 1, {5, 9, 5, -1}), 160) == PA_ERR_BAD_INDEX);
  contains("must be distinct");

  // query starts
  pa::HostInts cl4 = H(3, 1, {10, 4, 7});
  EXPECT(pa::check_query_starts(H(4, 1, {0, 3, 7, 12}), cl4, 12) == PA_OK);
  EXPECT(pa::check_query_starts(H(4, 1, {1, 3, 7, 12}), cl4, 12) == PA_ERR_BAD_INDEX);
  EXPECT(pa::check_query_starts(H(4, 1, {0, 3, 2, 12}), cl4, 12) == PA_ERR_BAD_INDEX);
  EXPECT(pa::check_query_starts(H(4, 1, {0, 3, 8, 12}), cl4, 12) == PA_ERR_BAD_INDEX);  // 5 rows, 4 tokens
  EXPECT(pa::check_query_starts(H(4, 1, {0, 3, 7, 11}), cl4, 12) == PA_ERR_BAD_INDEX);
  EXPECT(pa::check_query_starts(H(0, 1, {}), cl4, 0) == PA_OK);

  // block pairs
  EXPECT(pa::check_block_pairs(H(3, 2, {1, 2, 3, 4, -1, 2}), 10, 10, true) == PA_OK);  // the skipped pair is ignored
  EXPECT(pa::check_block_pairs(H(2, 2, {1, 2, 3, 2}), 10, 10, false) == PA_ERR_BAD_INDEX);
  EXPECT(pa::check_block_pairs(H(2, 2, {1, 2, 2, 5}), 10, 10, true) == PA_ERR_BAD_INDEX);
  EXPECT(pa::check_block_pairs(H(2, 2, {1, 2, 2, 5}), 10, 10, false) == PA_OK);
}

}  // namespace

int main() {
  abi_argument_checks();
  validation_checks();
  if (fails) {
    std::fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  std::printf("C ABI host-side sanitizer run: all checks clean\n");
  return 0;
}
