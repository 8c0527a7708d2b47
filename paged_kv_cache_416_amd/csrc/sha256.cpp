// SHA-256 (FIPS 180-4, sections 4.1.2, 5.1.1, 6.2) for the prefix cache's block digests: the
// lesson note "Week 22 Day 2", section 3.1, identifies prompt blocks by a cryptographic digest.
// The round constants and the initial hash value are computed from their definition (the first
// 32 bits of the fractional parts of the cube roots of the first 64 primes, and of the square
// roots of the first 8 primes) rather than typed in.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

namespace pkv {
namespace {

uint32_t g_k[64], g_h0[8];

uint32_t frac_bits(long double x) {
    const long double f = x - std::floor(x);
    return static_cast<uint32_t>(std::floor(std::ldexp(f, 32)));
}

void init_constants() {
    int primes[64], n = 0;
    for (int c = 2; n < 64; ++c) {
        bool prime = true;
        for (int i = 0; i < n && primes[i] * primes[i] <= c; ++i)
            if (c % primes[i] == 0) prime = false;
        if (prime) primes[n++] = c;
    }
    for (int i = 0; i < 64; ++i) g_k[i] = frac_bits(std::cbrt(static_cast<long double>(primes[i])));
    for (int i = 0; i < 8; ++i) g_h0[i] = frac_bits(std::sqrt(static_cast<long double>(primes[i])));
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void compress(uint32_t h[8], const uint8_t *block) {
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
        w[t] = (uint32_t(block[4 * t]) << 24) | (uint32_t(block[4 * t + 1]) << 16) | (uint32_t(block[4 * t + 2]) << 8) |
               uint32_t(block[4 * t + 3]);
    for (int t = 16; t < 64; ++t) {
        const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
        const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
        w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], k = h[7];
    for (int t = 0; t < 64; ++t) {
        const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
        const uint32_t ch = (e & f) ^ (~e & g);
        const uint32_t t1 = k + S1 + ch + g_k[t] + w[t];
        const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
        const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
        const uint32_t t2 = S0 + maj;
        k = g;
        g = f;
        f = e;
        e = d + t1;
        d = c;
        c = b;
        b = a;
        a = t1 + t2;
    }
    h[0] += a;
    h[1] += b;
    h[2] += c;
    h[3] += d;
    h[4] += e;
    h[5] += f;
    h[6] += g;
    h[7] += k;
}

}  // namespace

// Digest of n bytes: padding with a 1 bit, zeros and the 64-bit big-endian bit length to a
// multiple of 512 bits, then one compression per 64-byte block.
void sha256(const uint8_t *data, size_t n, uint8_t out[32]) {
    static std::once_flag once;
    std::call_once(once, init_constants);
    uint32_t h[8];
    std::memcpy(h, g_h0, sizeof h);
    size_t i = 0;
    for (; i + 64 <= n; i += 64) compress(h, data + i);
    uint8_t tail[128] = {};
    const size_t r = n - i;
    std::memcpy(tail, data + i, r);
    tail[r] = 0x80;
    const size_t total = r + 9 <= 64 ? 64 : 128;
    const uint64_t bits = static_cast<uint64_t>(n) * 8;
    for (int b = 0; b < 8; ++b) tail[total - 1 - b] = static_cast<uint8_t>(bits >> (8 * b));
    compress(h, tail);
    if (total == 128) compress(h, tail + 64);
    for (int j = 0; j < 8; ++j)
        for (int b = 0; b < 4; ++b) out[4 * j + b] = static_cast<uint8_t>(h[j] >> (24 - 8 * b));
}

}  // namespace pkv
