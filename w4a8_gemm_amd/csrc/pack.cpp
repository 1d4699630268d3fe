// Host-side weight packer: progressive two-level quantization and the
// gfx950 register layout.
//
// Progressive quantization is the weight side of QServe/QoQ (page "[Feature]
// Support W4A8KV4 Quantization(QServe/QoQ)", quoted abstract): weights go to
// int8 with a per-row scale first, then to uint4 per group with an integer
// step and zero, so the GEMM recovers the int8 operand with integer
// multiply-subtract only.  The exact constants (+-119, ceil for the step,
// round-half-even everywhere) are this library's reading of that text; the
// LiquidGEMM digest ("Метод") asks the same decode to be overflow-free, which
// the +-119 level-1 range guarantees.  Packing is offline: off the serving
// path, as in the FLUTE abstract's offline restructuring.
//
// Built with -ffp-contract=off: every fp32 step is one IEEE operation.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/w4a8.h"
#include "layout.h"

namespace {

using namespace w4a8;

// fp32 -> IEEE binary16 bits, round-half-to-even, by integer manipulation.
uint16_t half_bits_rne(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return uint16_t(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  if (ax >= 0x477FF000u) return uint16_t(sign | 0x7C00u);  // >= 65520 rounds to inf
  if (ax < 0x38800000u) {                                   // below 2^-14: subnormal
    int e = int(ax >> 23);
    if (e < 102) return uint16_t(sign);                     // below 2^-25
    uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    int shift = 126 - e;                                    // to units of 2^-24
    uint32_t q = mant >> shift, rem = mant & ((1u << shift) - 1), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return uint16_t(sign | q);
  }
  uint32_t h = (ax - 0x38000000u) >> 13;                    // rebias exponent, keep 10 bits
  uint32_t rem = ax & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
  return uint16_t(sign | h);
}

float half_to_float(uint16_t h) {
  uint32_t sign = uint32_t(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  uint32_t bits;
  if (e == 0) {
    if (m == 0) {
      bits = sign;
    } else {  // subnormal: m * 2^-24
      float v = float(m) * (1.0f / 16777216.0f);
      std::memcpy(&bits, &v, 4);
      bits |= sign;
    }
  } else if (e == 31) {
    bits = sign | 0x7F800000u | (m << 13);
  } else {
    bits = sign | ((e + 112u) << 23) | (m << 13);
  }
  float f;
  std::memcpy(&f, &bits, 4);
  return f;
}

// round-half-to-even of a / b for b > 0, in integers.
int div_rne(int a, int b) {
  int q = a / b, r = a % b;  // truncating division; r carries the sign of a
  int twice = 2 * (r < 0 ? -r : r);
  if (twice > b || (twice == b && (q & 1))) q += (a < 0) ? -1 : 1;
  return q;
}

int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Nearest codebook level to an int8 value, ties to the lower code.
uint8_t nearest_level(int v) {
  int best = 0, dist = 1 << 30;
  for (int j = 0; j < 16; ++j) {
    const int d = std::abs(int(kNfLevels[j]) - v);
    if (d < dist) {
      dist = d;
      best = j;
    }
  }
  return uint8_t(best);
}

// Quantize one row into logical codes q[k], and per-group z / s2 (codebook
// mode: level-1 int8, then the nearest level's code; no z / s2).
w4a8_status quantize_row(const float* w, int k, int ge, bool codebook, uint8_t* q, uint8_t* z,
                         uint8_t* s2, uint16_t* s1_bits, std::vector<int>& w8) {
  for (int i = 0; i < k; ++i)
    if (!std::isfinite(w[i])) return W4A8_ERR_NONFINITE;

  if (ge == k && !codebook) {  // per-channel: one uint4 step (fp16) and zero per row
    float lo = 0.0f, hi = 0.0f;
    for (int i = 0; i < k; ++i) {
      lo = std::min(lo, w[i]);
      hi = std::max(hi, w[i]);
    }
    float span = hi - lo;
    uint16_t sb = half_bits_rne(span / 15.0f);
    if ((sb & 0x7C00u) == 0x7C00u) return W4A8_ERR_RANGE;
    *s1_bits = sb;
    float sf = half_to_float(sb);
    s2[0] = 1;
    if (sf == 0.0f) {
      z[0] = 0;
      std::memset(q, 0, size_t(k));
      return W4A8_OK;
    }
    float r = 1.0f / sf;
    int zz = clampi(int(std::nearbyint(-lo * r)), 0, 15);
    z[0] = uint8_t(zz);
    for (int i = 0; i < k; ++i) q[i] = uint8_t(clampi(int(std::nearbyint(w[i] * r)) + zz, 0, 15));
    return W4A8_OK;
  }

  // level 1: symmetric int8 per row, range +-119
  float amax = 0.0f;
  for (int i = 0; i < k; ++i) amax = std::max(amax, std::fabs(w[i]));
  uint16_t sb = half_bits_rne(amax / 119.0f);
  if ((sb & 0x7C00u) == 0x7C00u) return W4A8_ERR_RANGE;
  *s1_bits = sb;
  float sf = half_to_float(sb);
  if (sf == 0.0f) {
    std::fill(w8.begin(), w8.begin() + k, 0);
  } else {
    float r = 1.0f / sf;
    for (int i = 0; i < k; ++i) w8[i] = clampi(int(std::nearbyint(w[i] * r)), -119, 119);
  }
  if (codebook) {
    for (int i = 0; i < k; ++i) q[i] = nearest_level(w8[i]);
    return W4A8_OK;
  }
  // level 2: uint4 per group with integer step and zero
  for (int g0 = 0, gi = 0; g0 < k; g0 += ge, ++gi) {
    int lo = 0, hi = 0;
    for (int i = g0; i < g0 + ge; ++i) {
      lo = std::min(lo, w8[i]);
      hi = std::max(hi, w8[i]);
    }
    int step = std::max(1, (hi - lo + 14) / 15);
    int zero = div_rne(-lo, step);
    z[gi] = uint8_t(zero);
    s2[gi] = uint8_t(step);
    for (int i = g0; i < g0 + ge; ++i) q[i] = uint8_t(clampi(div_rne(w8[i], step) + zero, 0, 15));
  }
  return W4A8_OK;
}

bool shape_ok(int n, int k, int g) {
  if (n <= 0 || k <= 0) return false;
  if (n % kColTile || k % kKBlock || k > W4A8_K_MAX) return false;
  if (g == 0 || g == k || g == kCodebookG) return true;
  if (g != 32 && g != 64 && g != 128) return false;
  return k % g == 0;
}

struct Header {
  char magic[8];
  uint32_t version;
  int32_t n, k, g;  // g == 0: per-channel; g == kCodebookG: codebook mode
  uint64_t q_off, meta_off, s1_off, total;
  int8_t levels[16];  // codebook mode: the level of each code (else zero)
};

}  // namespace

extern "C" size_t w4a8_packed_size(int n, int k, int g) {
  if (!shape_ok(n, k, g)) return 0;
  return sections(n, k, g).total;
}

extern "C" w4a8_status w4a8_pack(const float* w, int n, int k, int ldw, int g, void* blob,
                                 size_t blob_bytes, int n_threads) {
  if (!w || !blob || n <= 0 || k <= 0 || ldw < k || g < 0) return W4A8_ERR_INVALID_ARGUMENT;
  if (!shape_ok(n, k, g)) return W4A8_ERR_UNSUPPORTED;
  Sections sec = sections(n, k, g);
  if (blob_bytes < sec.total) return W4A8_ERR_BUFFER_TOO_SMALL;
  const bool codebook = g == kCodebookG;
  const int ge = codebook ? k : effective_group(k, g);
  const int groups = std::max(1, sec.groups);
  const int kblocks = k / kKBlock;

  uint8_t* base = static_cast<uint8_t*>(blob);
  std::memset(base, 0, sec.total);
  uint8_t* qsec = base + sec.q_off;
  uint8_t* msec = base + sec.meta_off;
  uint16_t* s1sec = reinterpret_cast<uint16_t*>(base + sec.s1_off);

  int tiles = n / kColTile;
  int threads = n_threads > 0 ? n_threads : int(std::thread::hardware_concurrency());
  threads = std::max(1, std::min(threads, tiles));
  std::atomic<int> next{0};
  std::atomic<int> first_error{W4A8_OK};

  auto worker = [&]() {
    std::vector<int> w8(static_cast<size_t>(k));
    std::vector<uint8_t> q(static_cast<size_t>(k));
    std::vector<uint8_t> z(static_cast<size_t>(groups)), s2(static_cast<size_t>(groups));
    for (;;) {
      int t = next.fetch_add(1);
      if (t >= tiles || first_error.load() != W4A8_OK) break;
      for (int r = 0; r < kColTile; ++r) {
        int row = t * kColTile + r;
        uint16_t s1b = 0;
        w4a8_status st = quantize_row(w + size_t(row) * size_t(ldw), k, ge, codebook, q.data(),
                                      z.data(), s2.data(), &s1b, w8);
        if (st != W4A8_OK) {
          int expected = W4A8_OK;
          first_error.compare_exchange_strong(expected, int(st));
          return;
        }
        s1sec[row] = s1b;
        for (int gi = 0; gi < sec.groups; ++gi)
          msec[meta_position(row, gi, sec.meta_row_bytes)] = uint8_t((z[gi] & 15u) | ((s2[gi] - 1u) << 4));
        for (int kk = 0; kk < k; ++kk) {
          size_t byte;
          int nib;
          q_position(row, kk, kblocks, &byte, &nib);
          qsec[byte] |= uint8_t(q[kk] << (4 * nib));
        }
      }
    }
  };
  std::vector<std::thread> pool;
  for (int i = 1; i < threads; ++i) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
  if (first_error.load() != W4A8_OK) {
    std::memset(base, 0, sec.total);
    return w4a8_status(first_error.load());
  }

  Header h;
  std::memset(&h, 0, sizeof(h));
  std::memcpy(h.magic, kMagic, 8);
  h.version = kLayoutVersion;
  h.n = n;
  h.k = k;
  h.g = codebook ? kCodebookG : ((ge == k) ? 0 : g);
  h.q_off = sec.q_off;
  h.meta_off = sec.meta_off;
  h.s1_off = sec.s1_off;
  h.total = sec.total;
  if (codebook) std::memcpy(h.levels, kNfLevels, 16);
  std::memcpy(base, &h, sizeof(h));
  return W4A8_OK;
}

extern "C" w4a8_status w4a8_blob_info(const void* blob, size_t blob_bytes, int* n, int* k, int* g) {
  if (!blob || !n || !k || !g) return W4A8_ERR_INVALID_ARGUMENT;
  if (blob_bytes < sizeof(Header)) return W4A8_ERR_LAYOUT;
  Header h;
  std::memcpy(&h, blob, sizeof(h));
  if (std::memcmp(h.magic, kMagic, 8) != 0 || h.version != kLayoutVersion) return W4A8_ERR_LAYOUT;
  if (!shape_ok(h.n, h.k, h.g)) return W4A8_ERR_LAYOUT;
  Sections sec = sections(h.n, h.k, h.g);
  if (h.total != sec.total || h.q_off != sec.q_off || h.meta_off != sec.meta_off ||
      h.s1_off != sec.s1_off || blob_bytes < sec.total)
    return W4A8_ERR_LAYOUT;
  *n = h.n;
  *k = h.k;
  *g = h.g;
  return W4A8_OK;
}

extern "C" w4a8_status w4a8_unpack(const void* blob, size_t blob_bytes, uint8_t* q, uint8_t* z,
                                   uint8_t* s2, uint16_t* s1) {
  int n, k, g;
  w4a8_status st = w4a8_blob_info(blob, blob_bytes, &n, &k, &g);
  if (st != W4A8_OK) return st;
  Sections sec = sections(n, k, g);
  const uint8_t* base = static_cast<const uint8_t*>(blob);
  const uint8_t* qsec = base + sec.q_off;
  const uint8_t* msec = base + sec.meta_off;
  const int kblocks = k / kKBlock;
  for (int row = 0; row < n; ++row) {
    if (q) {
      for (int kk = 0; kk < k; ++kk) {
        size_t byte;
        int nib;
        q_position(row, kk, kblocks, &byte, &nib);
        q[size_t(row) * k + kk] = uint8_t((qsec[byte] >> (4 * nib)) & 15u);
      }
    }
    for (int gi = 0; gi < sec.groups; ++gi) {
      uint8_t mb = msec[meta_position(row, gi, sec.meta_row_bytes)];
      if (z) z[size_t(row) * sec.groups + gi] = uint8_t(mb & 15u);
      if (s2) s2[size_t(row) * sec.groups + gi] = uint8_t((mb >> 4) + 1u);
    }
    if (s1) std::memcpy(&s1[row], base + sec.s1_off + 2 * size_t(row), 2);
  }
  return W4A8_OK;
}
