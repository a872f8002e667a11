// Driver for the host packer (ternary_hybrid_bit_amd/csrc/wal_host.cpp) built
// with AddressSanitizer and UndefinedBehaviorSanitizer.  It goes through the C
// ABI only (include/wal.h) and keeps every buffer it hands over in a heap
// block of exactly the size it declares, so that a read or write one byte
// outside is reported by the sanitizer:
//   - round trips pack -> verify -> inspect -> unpack over random shapes of
//     every format (2-bit and base-3 codes, k = 0/2/4/8 sites, fp16 and fp24
//     scales, 0..4 binary paths of rank 1..64), ragged row counts included;
//   - inputs pack must reject (bad trit, site, sign or factor entry, a scale
//     its format cannot hold, a short destination) with the documented
//     status, and nothing written for the code checks;
//   - blobs cut short, blobs with random bytes flipped, blobs whose planes
//     are corrupted under a re-stamped checksum (so that the code checks, not
//     the checksum, have to catch them) and headers with extreme fields;
//   - the INT3, INT4 and INT5 packers: round trips, rejected codes and
//     scales with the destination untouched, short buffers;
//   - the workspace-size queries and wal_status_str over every status.
// Exit status 0 and a last line "packer_fuzz: ok ..." mean that every check
// held; a sanitizer report aborts the process with a non-zero status.
#include "../../include/wal.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace {

int g_fail = 0;
long g_checks = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    ++g_checks;                                            \
    if (!(cond)) {                                         \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                   \
      std::fprintf(stderr, "\n");                          \
      if (++g_fail > 20) std::exit(1);                     \
    }                                                      \
  } while (0)

// splitmix64 (Steele, Lea and Flood, 2014): enough for test inputs.
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  uint32_t below(uint32_t n) { return (uint32_t)(next() % n); }
};

// A heap block of exactly n bytes (at least one, so that a zero-size block
// still has an address the sanitizer guards).
struct Block {
  uint8_t* p = nullptr;
  size_t n = 0;
  explicit Block(size_t bytes) : n(bytes) { p = static_cast<uint8_t*>(std::malloc(bytes ? bytes : 1)); }
  ~Block() { std::free(p); }
  Block(const Block&) = delete;
  Block& operator=(const Block&) = delete;
};

template <class T>
T* alloc(size_t count) {
  return static_cast<T*>(std::malloc(count ? count * sizeof(T) : 1));
}

// A scale that fp16 holds exactly: m * 2^e with |m| < 2^11 and a normal or
// zero result.
float exact_fp16(Rng& r) {
  const int m = (int)r.below(2047) - 1023;
  const int e = (int)r.below(12) - 20;
  return std::ldexp((float)m, e);
}
// A scale that the 24-bit format (upper three bytes of fp32) holds exactly.
float exact_fp24(Rng& r) {
  uint32_t b = (uint32_t)(r.next() & 0xFFFFFF00u);
  const uint32_t exp = (b >> 23) & 0xFF;
  if (exp == 0xFF) b &= ~(1u << 30);  // keep it finite
  float v;
  std::memcpy(&v, &b, 4);
  return v;
}

struct Logical {
  wal_desc d;
  uint64_t G = 0;
  int8_t* T = nullptr;
  uint8_t* pos = nullptr;
  int8_t* sign = nullptr;
  float* alpha = nullptr;
  float* beta = nullptr;
  int8_t* U = nullptr;
  int8_t* V = nullptr;
  float* s = nullptr;
  uint64_t nT() const { return (uint64_t)d.out * d.in; }
  uint64_t nS() const { return (uint64_t)d.out * G * d.k; }
  uint64_t nA() const { return (uint64_t)d.out * G; }
  uint64_t nU() const { return (uint64_t)d.n_paths * d.out * d.rank; }
  uint64_t nV() const { return (uint64_t)d.n_paths * d.in * d.rank; }
  uint64_t ns() const { return (uint64_t)d.n_paths * d.rank; }
  void allocate() {
    G = d.in / 128;
    T = alloc<int8_t>(nT());
    alpha = alloc<float>(nA());
    if (d.k) { pos = alloc<uint8_t>(nS()); sign = alloc<int8_t>(nS()); beta = alloc<float>(nA()); }
    if (d.n_paths) { U = alloc<int8_t>(nU()); V = alloc<int8_t>(nV()); s = alloc<float>(ns()); }
  }
  ~Logical() {
    std::free(T); std::free(pos); std::free(sign); std::free(alpha); std::free(beta);
    std::free(U); std::free(V); std::free(s);
  }
};

void random_logical(Rng& r, Logical& L) {
  for (uint64_t i = 0; i < L.nT(); ++i) L.T[i] = (int8_t)((int)r.below(3) - 1);
  const bool f16 = L.d.scale_fmt == WAL_SCALE_FP16;
  for (uint64_t i = 0; i < L.nA(); ++i) {
    L.alpha[i] = f16 ? exact_fp16(r) : exact_fp24(r);
    if (L.d.k) L.beta[i] = f16 ? exact_fp16(r) : exact_fp24(r);
  }
  const uint32_t k = L.d.k;
  for (uint64_t g = 0; g < L.d.out * L.G && k; ++g) {
    // k distinct positions in ascending order: a random subset of 0..127
    bool taken[128] = {};
    uint32_t got = 0;
    while (got < k) {
      const uint32_t p = r.below(128);
      if (!taken[p]) { taken[p] = true; ++got; }
    }
    uint32_t i = 0;
    for (uint32_t p = 0; p < 128; ++p)
      if (taken[p]) { L.pos[g * k + i] = (uint8_t)p; L.sign[g * k + i] = r.below(2) ? 1 : -1; ++i; }
  }
  for (uint64_t i = 0; i < L.nU(); ++i) L.U[i] = r.below(2) ? 1 : -1;
  for (uint64_t i = 0; i < L.nV(); ++i) L.V[i] = r.below(2) ? 1 : -1;
  for (uint64_t i = 0; i < L.ns(); ++i) L.s[i] = exact_fp16(r);
}

wal_desc random_desc(Rng& r) {
  static const uint32_t ks[4] = {0, 2, 4, 8};
  wal_desc d;
  d.out = 1 + r.below(37);
  d.in = 128 * (1 + r.below(5));
  d.k = ks[r.below(4)];
  d.n_paths = r.below(5);
  d.rank = d.n_paths ? 1 + r.below(64) : 0;
  d.trit_fmt = r.below(2) ? WAL_TRIT_BASE3 : WAL_TRIT_2BIT;
  d.scale_fmt = r.below(2) ? WAL_SCALE_FP24 : WAL_SCALE_FP16;
  return d;
}

int pack(const Logical& L, Block& blob, wal_info* info) {
  return wal_pack(&L.d, L.T, L.pos, L.sign, L.alpha, L.beta, L.U, L.V, L.s, blob.p, blob.n, info);
}

// Re-stamp the header checksum (wal.h: sum of (i + 1) * w_i over the u32
// words after the header, modulo 2^64).
void restamp(uint8_t* b, uint64_t total) {
  uint64_t acc = 0, idx = 1;
  for (uint64_t o = WAL_HEADER_BYTES; o + 4 <= total; o += 4, ++idx) {
    uint32_t w;
    std::memcpy(&w, b + o, 4);
    acc += idx * (uint64_t)w;
  }
  std::memcpy(b + 176, &acc, 8);
}

bool same_bits(const float* a, const float* b, uint64_t n) { return !n || std::memcmp(a, b, n * sizeof(float)) == 0; }

// Unpack into exact-size outputs and compare with the logical arrays.
void check_unpack(const Logical& L, const uint8_t* blob, size_t bytes) {
  Logical O;
  O.d = L.d;
  O.allocate();
  int st = wal_unpack(blob, bytes, O.T, O.pos, O.sign, O.alpha, O.beta, O.U, O.V, O.s);
  CHECK(st == WAL_OK, "unpack status %d", st);
  if (st) return;
  CHECK(!std::memcmp(O.T, L.T, L.nT()), "T differs");
  CHECK(same_bits(O.alpha, L.alpha, L.nA()), "alpha differs");
  if (L.d.k) {
    CHECK(!std::memcmp(O.pos, L.pos, L.nS()), "site positions differ");
    CHECK(!std::memcmp(O.sign, L.sign, L.nS()), "site signs differ");
    CHECK(same_bits(O.beta, L.beta, L.nA()), "beta differs");
  }
  if (L.d.n_paths) {
    CHECK(!std::memcmp(O.U, L.U, L.nU()), "U differs");
    CHECK(!std::memcmp(O.V, L.V, L.nV()), "V differs");
    CHECK(same_bits(O.s, L.s, L.ns()), "s differs");
  }
  // every output may be left out
  st = wal_unpack(blob, bytes, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  CHECK(st == WAL_OK, "unpack with no outputs: %d", st);
}

bool known_status(int st) { return st <= 0 && st >= WAL_ERR_UNSUPPORTED; }

// Copy the first n bytes of a blob into a block of exactly n bytes and run
// every reader on it.
void readers_on_prefix(const Logical& L, const Block& blob, size_t n) {
  Block cut(n);
  if (n) std::memcpy(cut.p, blob.p, n);
  wal_info f;
  const int si = wal_inspect(cut.p, n, &f);
  const int sv = wal_verify(cut.p, n);
  Logical O;
  O.d = L.d;
  O.allocate();
  const int su = wal_unpack(cut.p, n, O.T, O.pos, O.sign, O.alpha, O.beta, O.U, O.V, O.s);
  CHECK(si == WAL_ERR_BUFFER && sv == WAL_ERR_BUFFER && su == WAL_ERR_BUFFER,
        "prefix of %zu bytes: inspect %d verify %d unpack %d", n, si, sv, su);
}

// Unpack a blob that verified, into outputs sized from its own header.
void check_unpack_any(const Block& blob) {
  wal_info f;
  int st = wal_inspect(blob.p, blob.n, &f);
  CHECK(st == WAL_OK, "inspect of a verified blob: %d", st);
  if (st) return;
  Logical O;
  O.d = f.d;
  O.allocate();
  st = wal_unpack(blob.p, blob.n, O.T, O.pos, O.sign, O.alpha, O.beta, O.U, O.V, O.s);
  CHECK(st == WAL_OK, "unpack of a verified blob: %d", st);
}

// One plane byte changed under a re-stamped checksum; expect `want`.
void expect_plane(const Block& blob, const wal_info& f, uint64_t off, uint8_t value, int want, const char* what) {
  Block bad(blob.n);
  std::memcpy(bad.p, blob.p, blob.n);
  bad.p[off] = value;
  restamp(bad.p, f.total_bytes);
  const int st = wal_verify(bad.p, bad.n);
  CHECK(st == want, "%s: verify %d, expected %d", what, st, want);
  if (st == WAL_OK) check_unpack_any(bad);
  else {
    Logical O;
    O.d = f.d;
    O.allocate();
    const int su = wal_unpack(bad.p, bad.n, O.T, O.pos, O.sign, O.alpha, O.beta, O.U, O.V, O.s);
    CHECK(su == want, "%s: unpack %d, expected %d", what, su, want);
  }
}

void corrupt_planes(Rng& r, const Logical& L, const wal_info& f, const Block& blob) {
  const wal_desc& d = L.d;
  const uint32_t n = r.below(d.out);
  const uint64_t row = f.off_codes + (uint64_t)n * f.row_stride;
  if (d.trit_fmt == WAL_TRIT_2BIT) {
    const uint32_t j = r.below(d.in);
    const uint8_t b = blob.p[row + j / 4];
    const uint8_t cleared = (uint8_t)(b & ~(3u << (2 * (j % 4))));
    expect_plane(blob, f, row + j / 4, (uint8_t)(cleared | (2u << (2 * (j % 4)))), WAL_ERR_CODE, "2-bit code 10");
    expect_plane(blob, f, row + j / 4, cleared, WAL_OK, "2-bit code set to zero");
  } else {
    const uint64_t nb = (d.in + 4) / 5;
    expect_plane(blob, f, row + r.below((uint32_t)nb), (uint8_t)(243 + r.below(13)), WAL_ERR_CODE,
                 "base-3 byte above 242");
    // any byte below 243 is valid where all five trits lie inside the row
    expect_plane(blob, f, row + r.below((uint32_t)(nb - 1)), (uint8_t)r.below(243), WAL_OK, "base-3 byte in range");
    if (d.in % 5) {  // the last byte's digits past the row end must be zero trits
      const uint32_t live = d.in % 5;
      uint32_t v = 0, pw = 1;
      for (uint32_t i = 0; i < 5; ++i, pw *= 3) v += (i < live ? 1u : 2u) * pw;
      expect_plane(blob, f, row + nb - 1, (uint8_t)v, WAL_ERR_CODE, "base-3 trit past the row end");
    }
    if (f.row_stride > nb)
      expect_plane(blob, f, row + nb + r.below((uint32_t)(f.row_stride - nb)), 0x7A, WAL_ERR_CODE,
                   "base-3 pad byte");
  }
  if (d.k >= 2) {
    const uint64_t g = (uint64_t)n * f.groups + r.below(f.groups);
    const uint64_t at = f.off_sites + g * d.k;
    const uint32_t i = 1 + r.below(d.k - 1);
    const uint8_t prev = blob.p[at + i - 1] & 0x7F;
    expect_plane(blob, f, at + i, (uint8_t)(prev | (blob.p[at + i] & 0x80)), WAL_ERR_CODE, "repeated site");
    expect_plane(blob, f, at + i, (uint8_t)(blob.p[at + i] ^ 0x80), WAL_OK, "site sign flipped");
  }
  if (d.n_paths && d.rank % 8) {
    const uint32_t p = r.below(d.n_paths);
    const uint64_t ub = (d.rank + 7) / 8;
    const uint64_t at = f.off_U[p] + (uint64_t)n * ub + ub - 1;
    expect_plane(blob, f, at, (uint8_t)(blob.p[at] | (0x80u)), WAL_ERR_CODE, "U pad bit set");
  }
  // scales are any bit pattern: a changed scale still verifies
  expect_plane(blob, f, f.off_alpha + r.below((uint32_t)(d.out * f.groups)), (uint8_t)r.below(256), WAL_OK,
               "alpha byte changed");
}

// Headers that lie: each must be rejected with FORMAT or BUFFER, reading
// nothing past the block.
void bad_headers(Rng& r, const Block& blob) {
  struct Edit { uint32_t off, bytes; uint64_t value; int want; const char* what; };
  const Edit edits[] = {
      {0, 4, 0x314C4158u, WAL_ERR_FORMAT, "magic"},
      {4, 4, 2, WAL_ERR_FORMAT, "version"},
      {8, 4, 0, WAL_ERR_FORMAT, "out 0"},
      {8, 4, 0xFFFFFFFFu, WAL_ERR_FORMAT, "out 2^32-1"},
      {12, 4, 127, WAL_ERR_FORMAT, "in 127"},
      {12, 4, 0xFFFFFF80u, WAL_ERR_FORMAT, "in 2^32-128"},
      {16, 4, 3, WAL_ERR_FORMAT, "k 3"},
      {20, 4, 5, WAL_ERR_FORMAT, "5 paths"},
      {24, 4, 65, WAL_ERR_FORMAT, "rank 65"},
      {28, 4, 2, WAL_ERR_FORMAT, "trit format 2"},
      {32, 4, 7, WAL_ERR_FORMAT, "scale format 7"},
      {36, 4, 1, WAL_ERR_FORMAT, "row stride"},
      {40, 8, 1ull << 62, WAL_ERR_FORMAT, "total bytes"},
      {48, 8, 0, WAL_ERR_FORMAT, "codes offset"},
      {64, 8, 1ull << 40, WAL_ERR_FORMAT, "alpha offset"},
      {184 + 8 * (uint32_t)(r.below(9)), 1, 1, WAL_ERR_FORMAT, "reserved byte"},
  };
  for (const Edit& e : edits) {
    Block bad(blob.n);
    std::memcpy(bad.p, blob.p, blob.n);
    std::memcpy(bad.p + e.off, &e.value, e.bytes);
    wal_info f;
    const int si = wal_inspect(bad.p, bad.n, &f), sv = wal_verify(bad.p, bad.n);
    CHECK(si == e.want && sv == e.want, "header %s: inspect %d verify %d", e.what, si, sv);
  }
}

// A header that is consistent with itself but describes a matrix far larger
// than the block that holds it: BUFFER, with no read past the block.
void huge_header() {
  wal_desc d = {1u << 20, 1u << 20, 8, 4, 64, WAL_TRIT_2BIT, WAL_SCALE_FP24};
  wal_info f;
  CHECK(wal_packed_size(&d, &f) == WAL_OK, "packed_size of the huge shape");
  Block small(WAL_HEADER_BYTES + 4096);
  std::memset(small.p, 0, small.n);
  auto put32 = [&](uint32_t off, uint32_t v) { std::memcpy(small.p + off, &v, 4); };
  auto put64 = [&](uint32_t off, uint64_t v) { std::memcpy(small.p + off, &v, 8); };
  put32(0, 0x314C4157u); put32(4, 1);
  put32(8, d.out); put32(12, d.in); put32(16, d.k); put32(20, d.n_paths); put32(24, d.rank);
  put32(28, d.trit_fmt); put32(32, d.scale_fmt); put32(36, f.row_stride);
  put64(40, f.total_bytes); put64(48, f.off_codes); put64(56, f.off_sites);
  put64(64, f.off_alpha); put64(72, f.off_beta);
  for (uint32_t p = 0; p < WAL_MAX_PATHS; ++p) {
    put64(80 + 8 * p, f.off_V[p]); put64(112 + 8 * p, f.off_U[p]); put64(144 + 8 * p, f.off_s[p]);
  }
  wal_info g;
  CHECK(wal_inspect(small.p, small.n, &g) == WAL_ERR_BUFFER, "huge header: inspect");
  CHECK(wal_verify(small.p, small.n) == WAL_ERR_BUFFER, "huge header: verify");
  CHECK(wal_unpack(small.p, small.n, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
            WAL_ERR_BUFFER,
        "huge header: unpack");
}

// Inputs that pack must turn down.  Code errors are found before anything is
// written, so the destination must hold what it held before.
void pack_rejections(Rng& r) {
  for (int it = 0; it < 24; ++it) {
    Logical L;
    L.d = random_desc(r);
    if (L.d.k < 2) L.d.k = 4;
    if (!L.d.n_paths) { L.d.n_paths = 1; L.d.rank = 1 + r.below(64); }
    L.allocate();
    random_logical(r, L);
    wal_info f;
    wal_packed_size(&L.d, &f);
    Block dst(f.total_bytes);
    auto expect = [&](int want, bool untouched, const char* what) {
      std::memset(dst.p, 0xA5, dst.n);
      const int st = pack(L, dst, nullptr);
      CHECK(st == want, "pack with %s: %d, expected %d", what, st, want);
      if (untouched) {
        bool same = true;
        for (size_t i = 0; i < dst.n; ++i) same = same && dst.p[i] == 0xA5;
        CHECK(same, "pack with %s wrote to the destination", what);
      }
    };
    const uint64_t ti = r.below((uint32_t)L.nT());
    int8_t keep = L.T[ti];
    L.T[ti] = r.below(2) ? 2 : -2;
    expect(WAL_ERR_CODE, true, "a trit outside {-1, 0, 1}");
    L.T[ti] = keep;

    const uint64_t gi = r.below((uint32_t)(L.d.out * L.G));
    uint8_t* p = L.pos + gi * L.d.k;
    int8_t* sg = L.sign + gi * L.d.k;
    const uint32_t i = 1 + r.below(L.d.k - 1);
    uint8_t kp = p[i];
    p[i] = p[i - 1];
    expect(WAL_ERR_CODE, true, "a repeated site");
    p[i] = (uint8_t)(p[i - 1] - (p[i - 1] ? 1 : 0));
    if (p[i - 1]) expect(WAL_ERR_CODE, true, "sites out of order");
    p[i] = kp;
    kp = p[L.d.k - 1];
    p[L.d.k - 1] = (uint8_t)(128 + r.below(128));
    expect(WAL_ERR_CODE, true, "a site position past 127");
    p[L.d.k - 1] = kp;
    keep = sg[i];
    sg[i] = 0;
    expect(WAL_ERR_CODE, true, "a site sign of 0");
    sg[i] = keep;

    const uint64_t ui = r.below((uint32_t)L.nU()), vi = r.below((uint32_t)L.nV());
    keep = L.U[ui];
    L.U[ui] = 0;
    expect(WAL_ERR_CODE, true, "a U entry of 0");
    L.U[ui] = keep;
    keep = L.V[vi];
    L.V[vi] = 3;
    expect(WAL_ERR_CODE, true, "a V entry of 3");
    L.V[vi] = keep;

    const uint64_t ai = r.below((uint32_t)L.nA());
    float kf = L.alpha[ai];
    L.alpha[ai] = 1.0f / 3.0f;
    expect(WAL_ERR_INEXACT, false, "alpha 1/3");
    L.alpha[ai] = INFINITY;
    expect(WAL_ERR_INEXACT, false, "alpha inf");
    L.alpha[ai] = kf;
    kf = L.beta[ai];
    L.beta[ai] = NAN;
    expect(WAL_ERR_INEXACT, false, "beta nan");
    L.beta[ai] = kf;
    const uint64_t si = r.below((uint32_t)L.ns());
    kf = L.s[si];
    L.s[si] = 70000.0f;  // above the largest fp16
    expect(WAL_ERR_INEXACT, false, "s above fp16's range");
    L.s[si] = 1e-9f;  // below fp16's smallest subnormal
    expect(WAL_ERR_INEXACT, false, "s below fp16's range");
    L.s[si] = kf;
    if (L.d.scale_fmt == WAL_SCALE_FP16) {
      kf = L.alpha[ai];
      L.alpha[ai] = std::ldexp(1.5f, -24);  // half of the smallest fp16 subnormal
      expect(WAL_ERR_INEXACT, false, "alpha between fp16 subnormals");
      L.alpha[ai] = std::ldexp(1023.5f, -24);  // a half step below the largest subnormal
      expect(WAL_ERR_INEXACT, false, "alpha between the largest fp16 subnormals");
      L.alpha[ai] = std::ldexp(1023.0f, -24);  // the largest fp16 subnormal: exact
      expect(WAL_OK, false, "alpha the largest fp16 subnormal");
      L.alpha[ai] = std::ldexp(1.0f, -24);  // the smallest fp16 subnormal: exact
      expect(WAL_OK, false, "alpha the smallest fp16 subnormal");
      L.alpha[ai] = kf;
    }

    // one byte short, then the right size again
    {
      Block shortb(f.total_bytes - 1);
      const int st = wal_pack(&L.d, L.T, L.pos, L.sign, L.alpha, L.beta, L.U, L.V, L.s, shortb.p, shortb.n, nullptr);
      CHECK(st == WAL_ERR_BUFFER, "pack into a block one byte short: %d", st);
    }
    expect(WAL_OK, false, "the original inputs");
    CHECK(wal_verify(dst.p, dst.n) == WAL_OK, "verify after the rejections");

    // missing parts
    CHECK(wal_pack(&L.d, nullptr, L.pos, L.sign, L.alpha, L.beta, L.U, L.V, L.s, dst.p, dst.n, nullptr) ==
              WAL_ERR_ARG, "pack without T");
    CHECK(wal_pack(&L.d, L.T, nullptr, L.sign, L.alpha, L.beta, L.U, L.V, L.s, dst.p, dst.n, nullptr) ==
              WAL_ERR_ARG, "pack without sites");
    CHECK(wal_pack(&L.d, L.T, L.pos, L.sign, L.alpha, L.beta, nullptr, L.V, L.s, dst.p, dst.n, nullptr) ==
              WAL_ERR_ARG, "pack without U");
  }
  // descriptors outside the format
  wal_desc bad[] = {
      {0, 128, 0, 0, 0, WAL_TRIT_2BIT, WAL_SCALE_FP16},
      {4, 130, 0, 0, 0, WAL_TRIT_2BIT, WAL_SCALE_FP16},
      {4, 128, 6, 0, 0, WAL_TRIT_2BIT, WAL_SCALE_FP16},
      {4, 128, 0, 5, 8, WAL_TRIT_2BIT, WAL_SCALE_FP16},
      {4, 128, 0, 1, 0, WAL_TRIT_2BIT, WAL_SCALE_FP16},
      {4, 128, 0, 1, 65, WAL_TRIT_2BIT, WAL_SCALE_FP16},
      {4, 128, 0, 0, 3, WAL_TRIT_2BIT, WAL_SCALE_FP16},
      {0xFFFFFFFFu, 0xFFFFFF80u, 8, 4, 64, WAL_TRIT_2BIT, WAL_SCALE_FP16},
  };
  for (const wal_desc& d : bad) {
    wal_info f;
    CHECK(wal_packed_size(&d, &f) == WAL_ERR_SHAPE, "descriptor out %u in %u k %u paths %u rank %u", d.out, d.in,
          d.k, d.n_paths, d.rank);
  }
  wal_desc fmt = {4, 128, 0, 0, 0, 2, WAL_SCALE_FP16};
  wal_info f;
  CHECK(wal_packed_size(&fmt, &f) == WAL_ERR_ARG, "trit format 2");
  CHECK(wal_packed_size(nullptr, &f) == WAL_ERR_ARG, "NULL descriptor");
  CHECK(wal_inspect(nullptr, 4096, &f) == WAL_ERR_ARG, "inspect NULL");
  CHECK(wal_verify(nullptr, 4096) == WAL_ERR_ARG, "verify NULL");
}

typedef int (*qsize_fn)(uint32_t, uint32_t, size_t*);
typedef int (*qpack_fn)(uint32_t, uint32_t, const int8_t*, const float*, void*, size_t);
typedef int (*qunpack_fn)(uint32_t, uint32_t, const void*, size_t, int8_t*, float*);

void int_formats(Rng& r, int iters) {
  struct Fmt { int bits; qsize_fn size; qpack_fn pack; qunpack_fn unpack; };
  const Fmt fmts[3] = {{3, wal_int3_size, wal_int3_pack, wal_int3_unpack},
                       {4, wal_int4_size, wal_int4_pack, wal_int4_unpack},
                       {5, wal_int5_size, wal_int5_pack, wal_int5_unpack}};
  for (const Fmt& F : fmts) {
    const int lo = -(1 << (F.bits - 1)), hi = (1 << (F.bits - 1)) - 1;
    for (int it = 0; it < iters; ++it) {
      const uint32_t V = 1 + r.below(9), in = 128 * (1 + r.below(4)), G = in / 128;
      const uint64_t n = (uint64_t)V * in;
      size_t bytes = 0;
      CHECK(F.size(V, in, &bytes) == WAL_OK, "int%d size", F.bits);
      CHECK(bytes == n * F.bits / 8 + (uint64_t)V * G * 2, "int%d size %zu", F.bits, bytes);
      int8_t* q = alloc<int8_t>(n);
      float* s = alloc<float>((uint64_t)V * G);
      for (uint64_t i = 0; i < n; ++i) q[i] = (int8_t)(lo + (int)r.below((uint32_t)(hi - lo + 1)));
      for (uint64_t i = 0; i < (uint64_t)V * G; ++i) s[i] = exact_fp16(r);
      Block dst(bytes);
      CHECK(F.pack(V, in, q, s, dst.p, dst.n) == WAL_OK, "int%d pack", F.bits);
      int8_t* q2 = alloc<int8_t>(n);
      float* s2 = alloc<float>((uint64_t)V * G);
      CHECK(F.unpack(V, in, dst.p, dst.n, q2, s2) == WAL_OK, "int%d unpack", F.bits);
      CHECK(!std::memcmp(q, q2, n) && same_bits(s, s2, (uint64_t)V * G), "int%d round trip", F.bits);
      CHECK(F.unpack(V, in, dst.p, dst.n, nullptr, nullptr) == WAL_OK, "int%d unpack, no outputs", F.bits);
      {
        Block cut(bytes - 1);
        std::memcpy(cut.p, dst.p, cut.n);
        CHECK(F.unpack(V, in, cut.p, cut.n, q2, s2) == WAL_ERR_BUFFER, "int%d unpack one byte short", F.bits);
        CHECK(F.pack(V, in, q, s, cut.p, cut.n) == WAL_ERR_BUFFER, "int%d pack one byte short", F.bits);
      }
      // rejected inputs leave the destination as it was
      auto untouched = [&](int want, const char* what) {
        std::memset(dst.p, 0x5A, dst.n);
        const int st = F.pack(V, in, q, s, dst.p, dst.n);
        bool same = true;
        for (size_t i = 0; i < dst.n; ++i) same = same && dst.p[i] == 0x5A;
        CHECK(st == want && same, "int%d pack with %s: %d (untouched %d)", F.bits, what, st, (int)same);
      };
      const uint64_t qi = r.below((uint32_t)n);
      const int8_t kq = q[qi];
      q[qi] = (int8_t)(r.below(2) ? hi + 1 : lo - 1);
      untouched(WAL_ERR_CODE, "a code out of range");
      q[qi] = kq;
      const uint64_t si = r.below(V * G);
      const float ks = s[si];
      s[si] = 0.1f;
      untouched(WAL_ERR_INEXACT, "scale 0.1");
      s[si] = ks;
      CHECK(F.pack(V, in, nullptr, s, dst.p, dst.n) == WAL_ERR_ARG, "int%d pack without q", F.bits);
      CHECK(F.size(V, 100, &bytes) == WAL_ERR_SHAPE, "int%d in 100", F.bits);
      CHECK(F.size(0, in, &bytes) == WAL_ERR_ARG, "int%d V 0", F.bits);
      std::free(q); std::free(s); std::free(q2); std::free(s2);
    }
    // sizes at the bound are exact; past it (where V * in * bits would wrap
    // in 64 bits at the largest shapes) they are refused
    size_t big = 0;
    CHECK(F.size(1u << 20, 1u << 20, &big) == WAL_OK &&
              big == ((size_t)1 << 40) * F.bits / 8 + ((size_t)1 << 20) * ((1u << 20) / 128) * 2,
          "int%d size at V * in = 2^40", F.bits);
    CHECK(F.size((1u << 20) + 1, 1u << 20, &big) == WAL_ERR_SHAPE, "int%d size past 2^40", F.bits);
    CHECK(F.size(0xFFFFFFFFu, 0xFFFFFF80u, &big) == WAL_ERR_SHAPE, "int%d size of the largest shape", F.bits);
  }
}

void round_trips(Rng& r, int iters) {
  for (int it = 0; it < iters; ++it) {
    Logical L;
    L.d = random_desc(r);
    L.allocate();
    random_logical(r, L);
    wal_info f;
    int st = wal_packed_size(&L.d, &f);
    CHECK(st == WAL_OK, "packed_size %d", st);
    Block blob(f.total_bytes);
    wal_info g;
    st = pack(L, blob, &g);
    CHECK(st == WAL_OK, "pack %d (out %u in %u k %u paths %u rank %u fmt %u/%u)", st, L.d.out, L.d.in, L.d.k,
          L.d.n_paths, L.d.rank, L.d.trit_fmt, L.d.scale_fmt);
    if (st) continue;
    CHECK(!std::memcmp(&f, &g, sizeof f), "pack info differs from packed_size");
    CHECK(wal_verify(blob.p, blob.n) == WAL_OK, "verify of a fresh blob");
    wal_info h;
    CHECK(wal_inspect(blob.p, blob.n, &h) == WAL_OK && !std::memcmp(&f, &h, sizeof f), "inspect");
    check_unpack(L, blob.p, blob.n);

    size_t ws = 0;
    CHECK(wal_workspace_size(&f, 1, &ws) == WAL_OK && ws > 0, "workspace size");
    CHECK(wal_workspace_size(&f, 0, &ws) == WAL_ERR_ARG, "workspace size batch 0");
    CHECK(wal_prefill_workspace_size(&f, 1 + r.below(512), &ws) == WAL_OK, "prefill workspace size");

    // cut short: the header alone, part of it, all but one byte
    const size_t cuts[5] = {0, 1, WAL_HEADER_BYTES - 1, WAL_HEADER_BYTES, (size_t)f.total_bytes - 1};
    for (size_t c : cuts) readers_on_prefix(L, blob, c);
    readers_on_prefix(L, blob, WAL_HEADER_BYTES + r.below((uint32_t)(f.total_bytes - WAL_HEADER_BYTES)));

    // random bytes flipped anywhere: some status, never a fault
    for (int t = 0; t < 8; ++t) {
      Block bad(blob.n);
      std::memcpy(bad.p, blob.p, blob.n);
      const int flips = 1 + (int)r.below(4);
      for (int i = 0; i < flips; ++i) bad.p[r.below((uint32_t)bad.n)] ^= (uint8_t)(1 + r.below(255));
      wal_info x;
      const int si = wal_inspect(bad.p, bad.n, &x);
      const int sv = wal_verify(bad.p, bad.n);
      CHECK(known_status(si) && known_status(sv), "flip statuses %d %d", si, sv);
      if (sv == WAL_OK) check_unpack_any(bad);
    }

    // planes corrupted under a valid checksum: the code checks must see them
    corrupt_planes(r, L, f, blob);
    bad_headers(r, blob);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 0) : 1;
  const int iters = argc > 2 ? std::atoi(argv[2]) : 200;
  Rng r{seed};
  for (int st = 1; st >= -12; --st) CHECK(wal_status_str(st) != nullptr, "status string %d", st);
  round_trips(r, iters);
  huge_header();
  pack_rejections(r);
  int_formats(r, iters / 10 + 1);
  if (g_fail) {
    std::printf("packer_fuzz: %d of %ld checks failed\n", g_fail, g_checks);
    return 1;
  }
  std::printf("packer_fuzz: ok, %ld checks, seed %llu, %d shapes\n", g_checks, (unsigned long long)seed, iters);
  return 0;
}
