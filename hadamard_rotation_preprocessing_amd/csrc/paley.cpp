// Base Hadamard matrices of order K for the Kronecker form of widths that
// are not a power of two (AutoRound "Rotation Transform", section 1.5: such a
// width is split into a base order times a power of two and the base matrix
// is combined with a Sylvester block).
//
// The base matrices are Paley I matrices, built here from the finite-field
// definition: for q = p^r = 3 (mod 4), order K = q + 1,
//   H = I + [[0, 1^T], [-1, Q]],  Q[i][j] = chi(x_i - x_j),
// with chi the quadratic character of GF(q).  Field element i has base-p
// digits c_0 + c_1 p + ... as polynomial coefficients modulo the first monic
// irreducible polynomial of degree r in the order of the integer
// a_0 + a_1 p + ... + a_{r-1} p^{r-1}.  The order chosen for n is the
// smallest K = odd(n) * 2^j (j >= 0) dividing n with such a construction.
#include <stdint.h>

#include <cstddef>
#include <vector>

namespace hr {
namespace {

bool prime_power(int64_t q, int* p_out, int* r_out) {
    if (q < 2) return false;
    int64_t p = q;
    for (int64_t d = 2; d * d <= q; ++d)
        if (q % d == 0) {
            p = d;
            break;
        }
    int r = 0;
    int64_t t = q;
    while (t % p == 0) {
        t /= p;
        ++r;
    }
    if (t != 1) return false;
    *p_out = static_cast<int>(p);
    *r_out = r;
    return true;
}

// polynomial remainder of g modulo monic f over GF(p); returns true if zero
bool divides(const std::vector<int>& f, std::vector<int> g, int p) {
    const int df = static_cast<int>(f.size()) - 1;
    for (int d = static_cast<int>(g.size()) - 1; d >= df; --d) {
        const int c = ((g[d] % p) + p) % p;
        if (c)
            for (int k = 0; k <= df; ++k) g[d - df + k] = ((g[d - df + k] - c * f[k]) % p + p) % p;
    }
    for (int k = 0; k < df; ++k)
        if (g[k] % p) return false;
    return true;
}

int ipow(int b, int e) {
    int r = 1;
    while (e-- > 0) r *= b;
    return r;
}

std::vector<int> coeffs(int code, int p, int len) {
    std::vector<int> c(len);
    for (int k = 0; k < len; ++k) {
        c[k] = code % p;
        code /= p;
    }
    return c;
}

std::vector<int> field_modulus(int p, int r) {
    if (r == 1) return {0, 1};
    for (int code = 0; code < ipow(p, r); ++code) {
        std::vector<int> mod = coeffs(code, p, r);
        mod.push_back(1);
        bool irreducible = true;
        for (int deg = 1; deg <= r / 2 && irreducible; ++deg)
            for (int fc = 0; fc < ipow(p, deg) && irreducible; ++fc) {
                std::vector<int> f = coeffs(fc, p, deg);
                f.push_back(1);
                if (divides(f, mod, p)) irreducible = false;
            }
        if (irreducible) return mod;
    }
    return {};
}

}  // namespace

bool paley_exists(int64_t k) {
    int p, r;
    return k % 4 == 0 && prime_power(k - 1, &p, &r) && (k - 1) % 4 == 3;
}

// Fills h (k*k, row-major, +1/-1).  Returns false if no construction.
bool paley_matrix(int k, std::vector<int8_t>& h) {
    if (!paley_exists(k)) return false;
    const int q = k - 1;
    int p, r;
    prime_power(q, &p, &r);
    const std::vector<int> mod = field_modulus(p, r);
    // index -> coefficient vector; squares by multiplying polynomials
    std::vector<int> chi(q, -1);
    chi[0] = 0;
    for (int i = 1; i < q; ++i) {
        const std::vector<int> a = coeffs(i, p, r);
        std::vector<int> prod(2 * r - 1, 0);
        for (int x = 0; x < r; ++x)
            for (int y = 0; y < r; ++y) prod[x + y] = (prod[x + y] + a[x] * a[y]) % p;
        for (int d = 2 * r - 2; d >= r; --d) {
            const int c = prod[d];
            if (c)
                for (int t = 0; t <= r; ++t) prod[d - r + t] = ((prod[d - r + t] - c * mod[t]) % p + p) % p;
        }
        int idx = 0;
        for (int t = r - 1; t >= 0; --t) idx = idx * p + prod[t];
        chi[idx] = 1;
    }
    auto sub = [&](int i, int j) {
        int idx = 0, mul = 1;
        for (int t = 0; t < r; ++t) {
            const int d = ((i % p) - (j % p) + p) % p;
            idx += d * mul;
            mul *= p;
            i /= p;
            j /= p;
        }
        return idx;
    };
    h.assign(static_cast<size_t>(k) * k, 0);
    for (int i = 0; i < k; ++i)
        for (int j = 0; j < k; ++j) {
            int s;
            if (i == 0 && j == 0) s = 0;
            else if (i == 0) s = 1;
            else if (j == 0) s = -1;
            else s = chi[sub(i - 1, j - 1)];
            h[static_cast<size_t>(i) * k + j] = static_cast<int8_t>((i == j ? 1 : 0) + s);
        }
    return true;
}

// Smallest supported order K = odd(n) 2^j dividing n; 0 if none.
// For a prime q = k - 1 (= 3 mod 4): bit d of `bits` (d < q, words of 32)
// is set iff d is a nonzero square mod q.  The Paley I matrix is then
// H[r][c] = +1 for r == c or r == 0, -1 for c == 0 < r, and chi((r - c) mod
// q) otherwise (the construction above with field elements = integers mod
// q).  Returns false if q is not prime or the bits do not fit.
bool paley_character(int k, uint32_t* bits, int words) {
    int p, r;
    const int q = k - 1;
    if (!paley_exists(k) || !prime_power(q, &p, &r) || r != 1 || q > 32 * words) return false;
    for (int w = 0; w < words; ++w) bits[w] = 0u;
    for (int x = 1; x < q; ++x) {
        const int d = static_cast<int>((static_cast<int64_t>(x) * x) % q);
        bits[d >> 5] |= 1u << (d & 31);
    }
    return true;
}

int64_t kron_order(int64_t n) {
    if (n <= 0 || (n & (n - 1)) == 0) return 0;
    int64_t odd = n;
    while (odd % 2 == 0) odd /= 2;
    for (int64_t k = odd; n % k == 0; k *= 2)
        if (paley_exists(k)) return k;
    return 0;
}

}  // namespace hr
