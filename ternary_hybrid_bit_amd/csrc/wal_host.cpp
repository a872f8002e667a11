// Host side of libwal: blob layout, packer, validator and unpacker.
//
// The stored parts follow the WAL pages: packed ternary symbols, sparse
// positions/signs and fp16 scales in the executable cache (WAL-Ternary-8B
// card, executable-cache paragraph of "Install"), exactly k signed sites per
// group of 128 ("Representation"), 2-bit codes with three of four values used
// and a five-trits-per-byte base-3 container (WAL2-Ternary-27B card,
// "Что означает битность"), 24-bit float group scales and binary low-rank
// paths (WAL-Ternary-27B-RC1 card, "Representation").  The byte layout is
// documented in include/wal.h.  Validation is fail-closed, as the cards
// describe for their caches: anything malformed is rejected before use.
#include "wal_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace {

constexpr uint32_t kMagic = 0x314C4157u;  // "WAL1"
constexpr uint32_t kVersion = 1;
constexpr uint64_t kAlign = 256;
constexpr uint8_t kBase3Pad = 0x79;      // five zero trits (digits 1,1,1,1,1)
// Largest V * in of an INT3/4/5 matrix: its byte count, V * in * bits / 8,
// must not wrap in 64 bits (the ternary blobs have the same bound on out * in).
constexpr uint64_t kMaxQElems = 1ull << 40;

uint64_t up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

void put32(uint8_t* p, uint32_t v) { std::memcpy(p, &v, 4); }
void put64(uint8_t* p, uint64_t v) { std::memcpy(p, &v, 8); }
uint32_t get32(const uint8_t* p) { uint32_t v; std::memcpy(&v, p, 4); return v; }
uint64_t get64(const uint8_t* p) { uint64_t v; std::memcpy(&v, p, 8); return v; }

int check_desc(const wal_desc* d) {
  if (!d) return WAL_ERR_ARG;
  if (d->out == 0 || d->in == 0 || d->in % 128) return WAL_ERR_SHAPE;
  if (!(d->k == 0 || d->k == 2 || d->k == 4 || d->k == 8)) return WAL_ERR_SHAPE;
  if (d->n_paths > WAL_MAX_PATHS) return WAL_ERR_SHAPE;
  if (d->n_paths && (d->rank < 1 || d->rank > WAL_MAX_RANK)) return WAL_ERR_SHAPE;
  if (!d->n_paths && d->rank) return WAL_ERR_SHAPE;
  if (d->trit_fmt > WAL_TRIT_BASE3 || d->scale_fmt > WAL_SCALE_FP24) return WAL_ERR_ARG;
  // every offset below stays far inside 64 bits; keep rows addressable by u32
  if ((uint64_t)d->out * d->in > (1ull << 40)) return WAL_ERR_SHAPE;
  return WAL_OK;
}

uint32_t code_row_stride(uint32_t in, uint32_t fmt) {
  if (fmt == WAL_TRIT_2BIT) return in / 4;
  return (uint32_t)up((in + 4) / 5, 16);
}

void layout(const wal_desc* d, wal_info* f) {
  std::memset(f, 0, sizeof(*f));
  f->d = *d;
  f->groups = d->in / 128;
  f->row_stride = code_row_stride(d->in, d->trit_fmt);
  const uint64_t G = f->groups, out = d->out;
  const uint64_t sb = d->scale_fmt == WAL_SCALE_FP16 ? 2 : 3;
  uint64_t cur = WAL_HEADER_BYTES;
  f->off_codes = cur;
  cur = up(cur + out * f->row_stride, kAlign);
  if (d->k) { f->off_sites = cur; cur = up(cur + out * G * d->k, kAlign); }
  f->off_alpha = cur;
  cur = up(cur + out * G * sb, kAlign);
  if (d->k) { f->off_beta = cur; cur = up(cur + out * G * sb, kAlign); }
  for (uint32_t p = 0; p < d->n_paths; ++p) {
    f->off_V[p] = cur; cur = up(cur + (uint64_t)d->rank * (d->in / 8), kAlign);
    f->off_U[p] = cur; cur = up(cur + out * ((d->rank + 7) / 8), kAlign);
    f->off_s[p] = cur; cur = up(cur + 2ull * d->rank, kAlign);
  }
  f->total_bytes = cur;
  uint64_t codes = d->trit_fmt == WAL_TRIT_2BIT ? out * (d->in / 4) : out * ((d->in + 4) / 5);
  uint64_t alg = codes + out * G * d->k + out * G * sb * (d->k ? 2 : 1);
  alg += (uint64_t)d->n_paths * ((uint64_t)d->rank * (d->in / 8) + out * ((d->rank + 7) / 8) + 2ull * d->rank);
  f->algorithmic_bytes = alg;
}

// ---- scalar formats -------------------------------------------------------

// fp32 -> IEEE binary16 bits when the conversion is exact; false otherwise.
bool f32_to_f16_exact(float v, uint16_t* out) {
  uint32_t b;
  std::memcpy(&b, &v, 4);
  const uint32_t sign = (b >> 16) & 0x8000u;
  const int exp = (int)((b >> 23) & 0xFF);
  const uint32_t man = b & 0x7FFFFFu;
  if (exp == 0xFF) return false;                 // inf / nan are not scales
  if (exp == 0 && man == 0) { *out = (uint16_t)sign; return true; }
  if (exp == 0) return false;                    // fp32 subnormals underflow fp16
  const int e = exp - 127;                       // unbiased
  if (e > 15) return false;
  if (e >= -14) {                                // fp16 normal: 10 mantissa bits
    if (man & 0x1FFFu) return false;
    *out = (uint16_t)(sign | ((uint32_t)(e + 15) << 10) | (man >> 13));
    return true;
  }
  // fp16 subnormal: value = m * 2^-24 with m < 1024
  const int shift = -14 - e;                     // 1..
  if (shift > 10) return false;
  const uint32_t full = (man | 0x800000u);       // 24-bit significand
  const int drop = 13 + shift;
  if (full & ((1u << drop) - 1)) return false;
  *out = (uint16_t)(sign | (full >> drop));
  return true;
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  uint32_t b;
  if (e == 0) {
    if (m == 0) { b = sign; }
    else {                                       // subnormal: normalise
      int sh = 0;
      uint32_t mm = m;
      while (!(mm & 0x400)) { mm <<= 1; ++sh; }
      b = sign | ((uint32_t)(127 - 15 - sh + 1) << 23) | ((mm & 0x3FF) << 13);
    }
  } else if (e == 31) {
    b = sign | 0x7F800000u | (m << 13);
  } else {
    b = sign | ((e - 15 + 127) << 23) | (m << 13);
  }
  float v;
  std::memcpy(&v, &b, 4);
  return v;
}

int put_scale(uint8_t* dst, float v, uint32_t fmt) {
  if (fmt == WAL_SCALE_FP16) {
    uint16_t h;
    if (!f32_to_f16_exact(v, &h)) return WAL_ERR_INEXACT;
    std::memcpy(dst, &h, 2);
    return WAL_OK;
  }
  uint32_t b;
  std::memcpy(&b, &v, 4);
  if (b & 0xFFu) return WAL_ERR_INEXACT;
  if (((b >> 23) & 0xFF) == 0xFF) return WAL_ERR_INEXACT;
  dst[0] = (uint8_t)(b >> 8); dst[1] = (uint8_t)(b >> 16); dst[2] = (uint8_t)(b >> 24);
  return WAL_OK;
}

float get_scale(const uint8_t* src, uint32_t fmt) {
  if (fmt == WAL_SCALE_FP16) { uint16_t h; std::memcpy(&h, src, 2); return f16_to_f32(h); }
  uint32_t b = ((uint32_t)src[0] << 8) | ((uint32_t)src[1] << 16) | ((uint32_t)src[2] << 24);
  float v;
  std::memcpy(&v, &b, 4);
  return v;
}

uint64_t blob_checksum(const uint8_t* blob, uint64_t total) {
  uint64_t acc = 0, idx = 1;
  for (uint64_t o = WAL_HEADER_BYTES; o + 4 <= total; o += 4, ++idx) acc += idx * (uint64_t)get32(blob + o);
  return acc;
}

int read_header(const void* blob, size_t bytes, wal_info* info) {
  if (!blob || !info) return WAL_ERR_ARG;
  if (bytes < WAL_HEADER_BYTES) return WAL_ERR_BUFFER;
  const uint8_t* h = static_cast<const uint8_t*>(blob);
  if (get32(h) != kMagic || get32(h + 4) != kVersion) return WAL_ERR_FORMAT;
  for (int i = 184; i < 256; ++i) if (h[i]) return WAL_ERR_FORMAT;
  wal_desc d;
  d.out = get32(h + 8); d.in = get32(h + 12); d.k = get32(h + 16);
  d.n_paths = get32(h + 20); d.rank = get32(h + 24);
  d.trit_fmt = get32(h + 28); d.scale_fmt = get32(h + 32);
  if (check_desc(&d) != WAL_OK) return WAL_ERR_FORMAT;
  wal_info f;
  layout(&d, &f);
  bool ok = get32(h + 36) == f.row_stride && get64(h + 40) == f.total_bytes &&
            get64(h + 48) == f.off_codes && get64(h + 56) == f.off_sites &&
            get64(h + 64) == f.off_alpha && get64(h + 72) == f.off_beta;
  for (int p = 0; p < WAL_MAX_PATHS; ++p)
    ok = ok && get64(h + 80 + 8 * p) == f.off_V[p] && get64(h + 112 + 8 * p) == f.off_U[p] &&
         get64(h + 144 + 8 * p) == f.off_s[p];
  if (!ok) return WAL_ERR_FORMAT;
  if (bytes < f.total_bytes) return WAL_ERR_BUFFER;
  *info = f;
  return WAL_OK;
}

}  // namespace

namespace wal {
// A wal_info is trusted by the product calls only if it is exactly the
// layout its descriptor implies.
int check_info(const wal_info* info) {
  if (!info) return WAL_ERR_ARG;
  int st = check_desc(&info->d);
  if (st) return st;
  wal_info f;
  layout(&info->d, &f);
  bool same = f.row_stride == info->row_stride && f.groups == info->groups &&
              f.total_bytes == info->total_bytes && f.off_codes == info->off_codes &&
              f.off_sites == info->off_sites && f.off_alpha == info->off_alpha &&
              f.off_beta == info->off_beta && f.algorithmic_bytes == info->algorithmic_bytes;
  for (int p = 0; p < WAL_MAX_PATHS; ++p)
    same = same && f.off_V[p] == info->off_V[p] && f.off_U[p] == info->off_U[p] &&
           f.off_s[p] == info->off_s[p];
  if (!same) return WAL_ERR_FORMAT;
  return WAL_OK;
}
}  // namespace wal

extern "C" {

const char* wal_status_str(int s) {
  switch (s) {
    case WAL_OK: return "WAL_OK";
    case WAL_ERR_ARG: return "WAL_ERR_ARG: null pointer or argument out of range";
    case WAL_ERR_SHAPE: return "WAL_ERR_SHAPE: unsupported shape (in % 128, k, paths, rank)";
    case WAL_ERR_CODE: return "WAL_ERR_CODE: invalid trit, site, sign or factor entry";
    case WAL_ERR_INEXACT: return "WAL_ERR_INEXACT: scale not exactly representable in its storage format";
    case WAL_ERR_BUFFER: return "WAL_ERR_BUFFER: buffer too small";
    case WAL_ERR_ALIGN: return "WAL_ERR_ALIGN: misaligned device pointer";
    case WAL_ERR_FORMAT: return "WAL_ERR_FORMAT: bad magic, version, layout or checksum";
    case WAL_ERR_DEVICE: return "WAL_ERR_DEVICE: HIP launch or runtime failure";
    case WAL_ERR_UNSUPPORTED: return "WAL_ERR_UNSUPPORTED: valid input not handled by this build";
    default: return "WAL: unknown status";
  }
}

int wal_packed_size(const wal_desc* desc, wal_info* info) {
  int st = check_desc(desc);
  if (st) return st;
  if (!info) return WAL_ERR_ARG;
  layout(desc, info);
  return WAL_OK;
}

int wal_pack(const wal_desc* d, const int8_t* T, const uint8_t* site_pos, const int8_t* site_sign,
             const float* alpha, const float* beta, const int8_t* U, const int8_t* V,
             const float* s, void* dst_v, size_t dst_bytes, wal_info* info_out) {
  int st = check_desc(d);
  if (st) return st;
  if (!T || !alpha || !dst_v) return WAL_ERR_ARG;
  if (d->k && (!site_pos || !site_sign || !beta)) return WAL_ERR_ARG;
  if (d->n_paths && (!U || !V || !s)) return WAL_ERR_ARG;
  wal_info f;
  layout(d, &f);
  if (dst_bytes < f.total_bytes) return WAL_ERR_BUFFER;
  uint8_t* dst = static_cast<uint8_t*>(dst_v);
  const uint64_t out = d->out, in = d->in, G = f.groups, k = d->k, r = d->rank;

  // Validate every logical entry before writing anything.
  for (uint64_t i = 0; i < out * in; ++i)
    if (T[i] < -1 || T[i] > 1) return WAL_ERR_CODE;
  if (k) {
    for (uint64_t gi = 0; gi < out * G; ++gi) {
      const uint8_t* p = site_pos + gi * k;
      const int8_t* sg = site_sign + gi * k;
      for (uint64_t i = 0; i < k; ++i) {
        if (p[i] >= 128 || (sg[i] != 1 && sg[i] != -1)) return WAL_ERR_CODE;
        if (i && p[i] <= p[i - 1]) return WAL_ERR_CODE;
      }
    }
  }
  for (uint64_t i = 0; i < (uint64_t)d->n_paths * out * r; ++i)
    if (U[i] != 1 && U[i] != -1) return WAL_ERR_CODE;
  for (uint64_t i = 0; i < (uint64_t)d->n_paths * in * r; ++i)
    if (V[i] != 1 && V[i] != -1) return WAL_ERR_CODE;

  std::memset(dst, 0, f.total_bytes);
  // scales first: they are the only entries that can be inexact
  const uint64_t sb = d->scale_fmt == WAL_SCALE_FP16 ? 2 : 3;
  for (uint64_t i = 0; i < out * G; ++i) {
    if ((st = put_scale(dst + f.off_alpha + i * sb, alpha[i], d->scale_fmt))) return st;
    if (k && (st = put_scale(dst + f.off_beta + i * sb, beta[i], d->scale_fmt))) return st;
  }
  for (uint32_t p = 0; p < d->n_paths; ++p)
    for (uint64_t i = 0; i < r; ++i)
      if ((st = put_scale(dst + f.off_s[p] + 2 * i, s[p * r + i], WAL_SCALE_FP16))) return st;

  // codes
  for (uint64_t n = 0; n < out; ++n) {
    const int8_t* t = T + n * in;
    uint8_t* row = dst + f.off_codes + n * f.row_stride;
    if (d->trit_fmt == WAL_TRIT_2BIT) {
      for (uint64_t j = 0; j < in; j += 4) {
        uint8_t b = 0;
        for (int i = 0; i < 4; ++i) b |= (uint8_t)((uint8_t)t[j + i] & 3u) << (2 * i);
        row[j / 4] = b;
      }
    } else {
      const uint64_t nb = (in + 4) / 5;
      for (uint64_t m = 0; m < nb; ++m) {
        uint32_t v = 0, pw = 1;
        for (int i = 0; i < 5; ++i, pw *= 3) {
          const uint64_t j = 5 * m + i;
          const uint32_t digit = j < in ? (uint32_t)(t[j] + 1) : 1u;
          v += digit * pw;
        }
        row[m] = (uint8_t)v;
      }
      for (uint64_t m = nb; m < f.row_stride; ++m) row[m] = kBase3Pad;
    }
  }
  // sites
  if (k) {
    for (uint64_t i = 0; i < out * G * k; ++i)
      dst[f.off_sites + i] = (uint8_t)(site_pos[i] | (site_sign[i] < 0 ? 0x80 : 0));
  }
  // binary factors: set bit = -1, LSB first
  for (uint32_t p = 0; p < d->n_paths; ++p) {
    const int8_t* Up = U + (uint64_t)p * out * r;
    const int8_t* Vp = V + (uint64_t)p * in * r;
    const uint64_t ub = (r + 7) / 8;
    for (uint64_t n = 0; n < out; ++n)
      for (uint64_t q = 0; q < r; ++q)
        if (Up[n * r + q] < 0) dst[f.off_U[p] + n * ub + q / 8] |= (uint8_t)(1u << (q % 8));
    for (uint64_t q = 0; q < r; ++q)
      for (uint64_t j = 0; j < in; ++j)
        if (Vp[j * r + q] < 0) dst[f.off_V[p] + q * (in / 8) + j / 8] |= (uint8_t)(1u << (j % 8));
  }
  // header
  put32(dst + 0, kMagic); put32(dst + 4, kVersion);
  put32(dst + 8, d->out); put32(dst + 12, d->in); put32(dst + 16, d->k);
  put32(dst + 20, d->n_paths); put32(dst + 24, d->rank);
  put32(dst + 28, d->trit_fmt); put32(dst + 32, d->scale_fmt); put32(dst + 36, f.row_stride);
  put64(dst + 40, f.total_bytes); put64(dst + 48, f.off_codes); put64(dst + 56, f.off_sites);
  put64(dst + 64, f.off_alpha); put64(dst + 72, f.off_beta);
  for (int p = 0; p < WAL_MAX_PATHS; ++p) {
    put64(dst + 80 + 8 * p, f.off_V[p]);
    put64(dst + 112 + 8 * p, f.off_U[p]);
    put64(dst + 144 + 8 * p, f.off_s[p]);
  }
  put64(dst + 176, blob_checksum(dst, f.total_bytes));
  if (info_out) *info_out = f;
  return WAL_OK;
}

int wal_inspect(const void* blob, size_t bytes, wal_info* info) { return read_header(blob, bytes, info); }

int wal_verify(const void* blob, size_t bytes) {
  wal_info f;
  int st = read_header(blob, bytes, &f);
  if (st) return st;
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  if (blob_checksum(b, f.total_bytes) != get64(b + 176)) return WAL_ERR_FORMAT;
  const wal_desc& d = f.d;
  const uint64_t out = d.out, in = d.in, G = f.groups, k = d.k, r = d.rank;
  for (uint64_t n = 0; n < out; ++n) {
    const uint8_t* row = b + f.off_codes + n * f.row_stride;
    if (d.trit_fmt == WAL_TRIT_2BIT) {
      for (uint64_t j = 0; j < f.row_stride; ++j)
        for (int i = 0; i < 4; ++i)
          if (((row[j] >> (2 * i)) & 3) == 2) return WAL_ERR_CODE;
    } else {
      const uint64_t nb = (in + 4) / 5;
      for (uint64_t m = 0; m < nb; ++m) {
        if (row[m] > 242) return WAL_ERR_CODE;
        // digits past the row end must be zero trits
        uint32_t v = row[m];
        for (int i = 0; i < 5; ++i, v /= 3)
          if (5 * m + i >= in && v % 3 != 1) return WAL_ERR_CODE;
      }
      for (uint64_t m = nb; m < f.row_stride; ++m)
        if (row[m] != kBase3Pad) return WAL_ERR_CODE;
    }
  }
  if (k) {
    for (uint64_t gi = 0; gi < out * G; ++gi) {
      const uint8_t* p = b + f.off_sites + gi * k;
      for (uint64_t i = 1; i < k; ++i)
        if ((p[i] & 0x7F) <= (p[i - 1] & 0x7F)) return WAL_ERR_CODE;
    }
  }
  for (uint32_t p = 0; p < d.n_paths; ++p) {
    if (r % 8) {
      const uint64_t ub = (r + 7) / 8;
      const uint8_t mask = (uint8_t)(0xFFu << (r % 8));
      for (uint64_t n = 0; n < out; ++n)
        if (b[f.off_U[p] + n * ub + ub - 1] & mask) return WAL_ERR_CODE;
    }
  }
  return WAL_OK;
}

int wal_unpack(const void* blob, size_t bytes, int8_t* T, uint8_t* site_pos, int8_t* site_sign,
               float* alpha, float* beta, int8_t* U, int8_t* V, float* s) {
  int st = wal_verify(blob, bytes);
  if (st) return st;
  wal_info f;
  read_header(blob, bytes, &f);
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  const wal_desc& d = f.d;
  const uint64_t out = d.out, in = d.in, G = f.groups, k = d.k, r = d.rank;
  const uint64_t sb = d.scale_fmt == WAL_SCALE_FP16 ? 2 : 3;
  if (T) {
    for (uint64_t n = 0; n < out; ++n) {
      const uint8_t* row = b + f.off_codes + n * f.row_stride;
      int8_t* t = T + n * in;
      if (d.trit_fmt == WAL_TRIT_2BIT) {
        for (uint64_t j = 0; j < in; ++j) {
          const uint32_t c = (row[j / 4] >> (2 * (j % 4))) & 3u;
          t[j] = c == 3 ? -1 : (int8_t)c;
        }
      } else {
        for (uint64_t m = 0; 5 * m < in; ++m) {
          uint32_t v = row[m];
          for (uint64_t i = 0; i < 5; ++i, v /= 3)
            if (5 * m + i < in) t[5 * m + i] = (int8_t)((int)(v % 3) - 1);
        }
      }
    }
  }
  if (alpha)
    for (uint64_t i = 0; i < out * G; ++i) alpha[i] = get_scale(b + f.off_alpha + i * sb, d.scale_fmt);
  if (k) {
    if (beta)
      for (uint64_t i = 0; i < out * G; ++i) beta[i] = get_scale(b + f.off_beta + i * sb, d.scale_fmt);
    for (uint64_t i = 0; i < out * G * k; ++i) {
      const uint8_t v = b[f.off_sites + i];
      if (site_pos) site_pos[i] = v & 0x7F;
      if (site_sign) site_sign[i] = (v & 0x80) ? -1 : 1;
    }
  }
  for (uint32_t p = 0; p < d.n_paths; ++p) {
    const uint64_t ub = (r + 7) / 8;
    if (U)
      for (uint64_t n = 0; n < out; ++n)
        for (uint64_t q = 0; q < r; ++q)
          U[((uint64_t)p * out + n) * r + q] = (b[f.off_U[p] + n * ub + q / 8] >> (q % 8)) & 1 ? -1 : 1;
    if (V)
      for (uint64_t j = 0; j < in; ++j)
        for (uint64_t q = 0; q < r; ++q)
          V[((uint64_t)p * in + j) * r + q] = (b[f.off_V[p] + q * (in / 8) + j / 8] >> (j % 8)) & 1 ? -1 : 1;
    if (s)
      for (uint64_t q = 0; q < r; ++q) s[p * r + q] = get_scale(b + f.off_s[p] + 2 * q, WAL_SCALE_FP16);
  }
  return WAL_OK;
}

int wal_workspace_size(const wal_info* info, uint32_t batch, size_t* bytes) {
  if (!info || !bytes) return WAL_ERR_ARG;
  if (batch == 0 || batch > WAL_MAX_BATCH) return WAL_ERR_ARG;
  const int st = wal::check_info(info);
  if (st) return st;
  // z_p[r] for every path, rank and batch column and the partial sums of the
  // small-batch kernels (wal_gemv uses the first part only)
  *bytes = (size_t)wal::gemm_shape(*info, batch).bytes;
  return WAL_OK;
}

int wal_int4_size(uint32_t V, uint32_t in, size_t* bytes) {
  if (!bytes || !V || !in) return WAL_ERR_ARG;
  if (in % 128 || (uint64_t)V * in > kMaxQElems) return WAL_ERR_SHAPE;
  *bytes = (size_t)V * in / 2 + (size_t)V * (in / 128) * 2;
  return WAL_OK;
}

int wal_int4_pack(uint32_t V, uint32_t in, const int8_t* q, const float* s, void* dst, size_t dst_bytes) {
  size_t need = 0;
  int st = wal_int4_size(V, in, &need);
  if (st) return st;
  if (!q || !s || !dst) return WAL_ERR_ARG;
  if (dst_bytes < need) return WAL_ERR_BUFFER;
  const uint64_t n = (uint64_t)V * in, G = in / 128;
  for (uint64_t i = 0; i < n; ++i)
    if (q[i] < -8 || q[i] > 7) return WAL_ERR_CODE;
  uint8_t h[2];
  for (uint64_t i = 0; i < (uint64_t)V * G; ++i)   // every scale checked before anything is written
    if ((st = put_scale(h, s[i], WAL_SCALE_FP16))) return st;
  uint8_t* b = static_cast<uint8_t*>(dst);
  uint8_t* sc = b + n / 2;
  for (uint64_t i = 0; i < (uint64_t)V * G; ++i) (void)put_scale(sc + 2 * i, s[i], WAL_SCALE_FP16);
  for (uint64_t i = 0; i < n / 2; ++i)
    b[i] = (uint8_t)(((uint8_t)q[2 * i] & 0xFu) | (((uint8_t)q[2 * i + 1] & 0xFu) << 4));
  return WAL_OK;
}

int wal_int4_unpack(uint32_t V, uint32_t in, const void* src, size_t src_bytes, int8_t* q, float* s) {
  size_t need = 0;
  int st = wal_int4_size(V, in, &need);
  if (st) return st;
  if (!src) return WAL_ERR_ARG;
  if (src_bytes < need) return WAL_ERR_BUFFER;
  const uint64_t n = (uint64_t)V * in, G = in / 128;
  const uint8_t* b = static_cast<const uint8_t*>(src);
  if (q)
    for (uint64_t i = 0; i < n; ++i) {
      const uint32_t nib = (b[i / 2] >> (4 * (i & 1))) & 0xFu;
      q[i] = (int8_t)(nib >= 8 ? (int)nib - 16 : (int)nib);
    }
  if (s)
    for (uint64_t i = 0; i < (uint64_t)V * G; ++i) s[i] = get_scale(b + n / 2 + 2 * i, WAL_SCALE_FP16);
  return WAL_OK;
}

// INT3 and INT5 matrices: every row's b-bit codes as one bit stream (element j
// at stream bits b j .. b j + b - 1, LSB first), then fp16 scales per 128.
// A row is in * b / 8 whole bytes (in is a multiple of 128), so the rows'
// streams simply follow each other.
static int qstream_size(uint32_t bits, uint32_t V, uint32_t in, size_t* bytes) {
  if (!bytes || !V || !in) return WAL_ERR_ARG;
  if (in % 128 || (uint64_t)V * in > kMaxQElems) return WAL_ERR_SHAPE;
  *bytes = (size_t)V * in * bits / 8 + (size_t)V * (in / 128) * 2;
  return WAL_OK;
}

static int qstream_pack(uint32_t bits, uint32_t V, uint32_t in, const int8_t* q, const float* s, void* dst,
                        size_t dst_bytes) {
  size_t need = 0;
  int st = qstream_size(bits, V, in, &need);
  if (st) return st;
  if (!q || !s || !dst) return WAL_ERR_ARG;
  if (dst_bytes < need) return WAL_ERR_BUFFER;
  const int lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
  const uint64_t n = (uint64_t)V * in, G = in / 128, cb = n * bits / 8;
  for (uint64_t i = 0; i < n; ++i)
    if (q[i] < lo || q[i] > hi) return WAL_ERR_CODE;
  uint8_t h[2];
  for (uint64_t i = 0; i < (uint64_t)V * G; ++i)   // every scale checked before anything is written
    if ((st = put_scale(h, s[i], WAL_SCALE_FP16))) return st;
  uint8_t* b = static_cast<uint8_t*>(dst);
  std::memset(b, 0, cb);
  const uint32_t mask = (1u << bits) - 1u;
  for (uint64_t i = 0; i < n; ++i) {
    const uint32_t code = (uint32_t)q[i] & mask;
    for (uint32_t k = 0; k < bits; ++k)
      if ((code >> k) & 1u) b[(bits * i + k) / 8] |= (uint8_t)(1u << ((bits * i + k) % 8));
  }
  for (uint64_t i = 0; i < (uint64_t)V * G; ++i) (void)put_scale(b + cb + 2 * i, s[i], WAL_SCALE_FP16);
  return WAL_OK;
}

static int qstream_unpack(uint32_t bits, uint32_t V, uint32_t in, const void* src, size_t src_bytes, int8_t* q,
                          float* s) {
  size_t need = 0;
  int st = qstream_size(bits, V, in, &need);
  if (st) return st;
  if (!src) return WAL_ERR_ARG;
  if (src_bytes < need) return WAL_ERR_BUFFER;
  const uint64_t n = (uint64_t)V * in, G = in / 128, cb = n * bits / 8;
  const uint8_t* b = static_cast<const uint8_t*>(src);
  if (q)
    for (uint64_t i = 0; i < n; ++i) {
      uint32_t code = 0;
      for (uint32_t k = 0; k < bits; ++k) code |= ((b[(bits * i + k) / 8] >> ((bits * i + k) % 8)) & 1u) << k;
      q[i] = (int8_t)(code >> (bits - 1) ? (int)code - (1 << bits) : (int)code);
    }
  if (s)
    for (uint64_t i = 0; i < (uint64_t)V * G; ++i) s[i] = get_scale(b + cb + 2 * i, WAL_SCALE_FP16);
  return WAL_OK;
}

int wal_int3_size(uint32_t V, uint32_t in, size_t* bytes) { return qstream_size(3, V, in, bytes); }
int wal_int3_pack(uint32_t V, uint32_t in, const int8_t* q, const float* s, void* dst, size_t dst_bytes) {
  return qstream_pack(3, V, in, q, s, dst, dst_bytes);
}
int wal_int3_unpack(uint32_t V, uint32_t in, const void* src, size_t src_bytes, int8_t* q, float* s) {
  return qstream_unpack(3, V, in, src, src_bytes, q, s);
}
int wal_int5_size(uint32_t V, uint32_t in, size_t* bytes) { return qstream_size(5, V, in, bytes); }
int wal_int5_pack(uint32_t V, uint32_t in, const int8_t* q, const float* s, void* dst, size_t dst_bytes) {
  return qstream_pack(5, V, in, q, s, dst, dst_bytes);
}
int wal_int5_unpack(uint32_t V, uint32_t in, const void* src, size_t src_bytes, int8_t* q, float* s) {
  return qstream_unpack(5, V, in, src, src_bytes, q, s);
}

int wal_prefill_workspace_size(const wal_info* info, uint32_t batch, size_t* bytes) {
  if (!info || !bytes) return WAL_ERR_ARG;
  if (batch == 0 || batch > WAL_MAX_PREFILL_BATCH) return WAL_ERR_ARG;
  const int st = wal::check_info(info);
  if (st) return st;
  *bytes = (size_t)wal::prefill_shape(*info, batch).bytes;
  return WAL_OK;
}

}  // extern "C"

namespace wal {

PrefillShape prefill_shape(const wal_info& f, uint32_t batch) {
  PrefillShape S;
  const uint32_t rows = prefill_rows(f.d.scale_fmt);
  S.rblocks = (f.d.out + rows - 1) / rows;
  S.chunks = (batch + kPrefillCols - 1) / kPrefillCols;
  S.sweeps = (f.groups + kPrefillSweepGroups - 1) / kPrefillSweepGroups;
  const uint64_t base = (uint64_t)S.rblocks * S.chunks;
  S.nsplit = 1;
  if (base < kPrefillTiles) S.nsplit = (uint32_t)std::min<uint64_t>(S.sweeps, (kPrefillTiles + base - 1) / base);
  S.cgw = std::min<uint32_t>(8, S.chunks);
  const uint64_t ngroups = (S.chunks + S.cgw - 1) / S.cgw;
  const uint64_t ids = ngroups * S.rblocks * S.nsplit * S.cgw;
  S.per_xcd = (uint32_t)((ids + 7) / 8);
  S.tiles = (uint32_t)ids;
  {
    const uint64_t tiles = std::max<uint64_t>(1, (uint64_t)((batch + 15) / 16) * ((f.d.n_paths * f.d.rank + 15) / 16));
    uint64_t splits = std::max<uint64_t>(1, (kZmmaWaves + tiles - 1) / tiles);
    splits = std::min<uint64_t>(std::min<uint64_t>(splits, kZmmaMaxSplits), f.groups);
    S.zgroups = (uint32_t)((f.groups + splits - 1) / splits);
    S.zc = (f.groups + S.zgroups - 1) / S.zgroups;
  }
  const uint64_t terms = (uint64_t)f.d.n_paths * f.d.rank;
  S.off_p = up(4 * terms * batch * S.zc, 256);
  S.bytes = S.off_p + (S.nsplit > 1 ? up(4ull * S.nsplit * batch * f.d.out, 256) : 0);
  return S;
}

GemmShape gemm_shape(const wal_info& f, uint32_t batch) {
  GemmShape S;
  const uint64_t terms = (uint64_t)f.d.n_paths * f.d.rank;
  S.nt = (batch + 15) / 16;
  S.passes = (f.d.in + kPass2bit - 1) / kPass2bit;
  S.zc = (f.d.in + kZChunkCols - 1) / kZChunkCols;
  S.slices = (f.d.in + kSliceCols - 1) / kSliceCols;
  S.off_cnt = kSyncBytes;
  S.off_z = kWsZeroBytes;
  // the small-batch kernels' fp32 partials per 4096 columns, or the single
  // product's tagged partials (8 bytes) per kZSingleCols columns
  const uint64_t zsmall = 4 * terms * batch * S.zc;
  const uint64_t zsingle = 8 * terms * ((f.d.in + kZSingleCols - 1) / kZSingleCols);
  S.off_p = S.off_z + up(zsmall > zsingle ? zsmall : zsingle, 256);
  S.bytes = S.off_p + up(4ull * S.slices * batch * f.d.out, 256);
  return S;
}

}  // namespace wal
