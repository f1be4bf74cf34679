// C-ABI entry points: argument validation, launch planning, dispatch.
//
// Every check runs before anything is enqueued, so a failing call leaves all
// outputs untouched (the all-or-nothing convention of the AIMET SpinQuant
// page: validate every pass, then mutate).  No silent fallback exists: a
// shape the kernels do not cover returns HR_EUNSUPPORTED.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <cmath>
#include <string>
#include <vector>

#include "../../include/hadarot.h"
#include "plan.h"

namespace hr {
bool paley_matrix(int k, std::vector<int8_t>& h);
bool paley_character(int k, uint32_t* bits, int words);
int64_t kron_order(int64_t n);
}  // namespace hr

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

int ok() {
    g_err.clear();
    return HR_OK;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int64_t v) {
    int l = 0;
    while ((int64_t{1} << l) < v) ++l;
    return l;
}

size_t dtype_size(int dt) { return dt == HR_F32 ? 4 : (dt == HR_BF16 ? 2 : 1); }

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// Validated quantizer spec.
struct QSpec {
    int format, sym, logg, scale_dtype;
    int64_t g;
    float tscale;  // NVFP4 tensor scale (1 otherwise)
};

int check_qspec(const hr_qspec* q, int64_t n, QSpec* out) {
    if (!q) return fail(HR_EINVAL, "quantizer spec is NULL");
    if (q->format != HR_Q_INT && q->format != HR_Q_MXFP4 && q->format != HR_Q_NVFP4)
        return fail(HR_EINVAL, "quantizer format %d is not HR_Q_INT, HR_Q_MXFP4 or HR_Q_NVFP4", q->format);
    if (q->bits != 4) return fail(HR_EUNSUPPORTED, "bits = %d: only 4-bit codes are implemented", q->bits);
    const int64_t g = q->group_size;
    float tscale = 1.0f;
    if (q->format == HR_Q_MXFP4) {
        if (g != 32) return fail(HR_EINVAL, "MXFP4 requires group_size 32 (got %lld)", (long long)g);
        if (q->scale_dtype != HR_E8M0) return fail(HR_EINVAL, "MXFP4 requires scale_dtype HR_E8M0");
    } else if (q->format == HR_Q_NVFP4) {
        if (g != 16) return fail(HR_EINVAL, "NVFP4 requires group_size 16 (got %lld)", (long long)g);
        if (q->scale_dtype != HR_E4M3) return fail(HR_EINVAL, "NVFP4 requires scale_dtype HR_E4M3");
        const float t = q->tensor_scale;
        if (!(t >= 0.0f) || !std::isfinite(t))
            return fail(HR_EINVAL, "NVFP4 tensor_scale must be positive and finite (0 means 1)");
        // denormal tensor scales would flush to zero in the kernels
        if (t != 0.0f && t < 1.17549435e-38f) return fail(HR_EINVAL, "NVFP4 tensor_scale is below the float range");
        tscale = t == 0.0f ? 1.0f : t;
    } else {
        if (g <= 0 || g % 2) return fail(HR_EINVAL, "group_size %lld must be positive and even", (long long)g);
        if (q->sym != 0 && q->sym != 1) return fail(HR_EINVAL, "sym must be 0 or 1");
        if (q->scale_dtype != HR_F32 && q->scale_dtype != HR_BF16)
            return fail(HR_EINVAL, "INT scales must be HR_F32 or HR_BF16");
    }
    if (n % g) return fail(HR_EINVAL, "group_size %lld does not divide n = %lld", (long long)g, (long long)n);
    if (!is_pow2(g)) return fail(HR_EUNSUPPORTED, "group_size %lld is not a power of two", (long long)g);
    out->format = q->format;
    out->sym = q->format == HR_Q_INT ? q->sym : 1;
    out->g = g;
    out->logg = ilog2(g);
    out->scale_dtype = q->format == HR_Q_MXFP4 ? 2 : (q->format == HR_Q_NVFP4 ? 3 : (q->scale_dtype == HR_BF16 ? 1 : 0));
    out->tscale = tscale;
    return HR_OK;
}

int check_shape(int dtype, int64_t rows, int64_t n) {
    if (dtype != HR_F32 && dtype != HR_BF16) return fail(HR_EINVAL, "dtype %d is not HR_F32 or HR_BF16", dtype);
    if (rows < 0) return fail(HR_EINVAL, "rows = %lld is negative", (long long)rows);
    if (n <= 0) return fail(HR_EINVAL, "n = %lld must be positive", (long long)n);
    if (n > (int64_t{1} << 40) || (rows > 0 && rows > (int64_t{1} << 50) / n))
        return fail(HR_EINVAL, "tensor too large (rows = %lld, n = %lld)", (long long)rows, (long long)n);
    return HR_OK;
}

// Rotation geometry: Sylvester block or Kronecker factorisation.
struct Geometry {
    int logb;       // log2 of the Hadamard block (Sylvester) or of M (Kronecker)
    int kron_k;     // 0 or the base order
    int64_t block;  // B (Sylvester) or M (Kronecker)
    float norm;
};

int check_block(int64_t n, int64_t block, Geometry* g) {
    g->kron_k = 0;
    if (block > 0 && block != n) {
        if (!is_pow2(block)) return fail(HR_EINVAL, "block %lld is not a power of two", (long long)block);
        if (n % block) return fail(HR_EINVAL, "block %lld does not divide n = %lld", (long long)block, (long long)n);
        if (block > 32768) return fail(HR_EUNSUPPORTED, "block %lld exceeds 32768", (long long)block);
        g->block = block;
        g->logb = ilog2(block);
        g->norm = static_cast<float>(1.0 / sqrt(static_cast<double>(block)));
        return HR_OK;
    }
    if (is_pow2(n)) {
        if (n > 32768) return fail(HR_EUNSUPPORTED, "full-width rotation of n = %lld exceeds 32768", (long long)n);
        g->block = n;
        g->logb = ilog2(n);
        g->norm = static_cast<float>(1.0 / sqrt(static_cast<double>(n)));
        return HR_OK;
    }
    const int64_t k = hr::kron_order(n);
    if (k == 0) return fail(HR_EUNSUPPORTED, "no supported base Hadamard order for n = %lld", (long long)n);
    if (k > hr::kMaxKron)
        return fail(HR_EUNSUPPORTED, "Kronecker base order %lld for n = %lld exceeds %d", (long long)k,
                    (long long)n, hr::kMaxKron);
    if (k > hr::kMaxKronDense) {
        uint32_t chi[hr::kMaxKron / 32];
        if (!hr::paley_character(static_cast<int>(k), chi, hr::kMaxKron / 32))
            return fail(HR_EUNSUPPORTED, "Kronecker base order %lld for n = %lld: orders above %d need a prime q = K - 1",
                        (long long)k, (long long)n, hr::kMaxKronDense);
    }
    if (n > 32768) return fail(HR_EUNSUPPORTED, "Kronecker rotation of n = %lld exceeds 32768", (long long)n);
    g->kron_k = static_cast<int>(k);
    g->block = n / k;
    g->logb = ilog2(g->block);
    g->norm = static_cast<float>(1.0 / sqrt(static_cast<double>(n)));
    return HR_OK;
}

int check_ptr(const void* p, const char* name, size_t align) {
    if (!p) return fail(HR_EINVAL, "%s is NULL", name);
    if (reinterpret_cast<uintptr_t>(p) % align)
        return fail(HR_EINVAL, "%s is not %zu-byte aligned", name, align);
    return HR_OK;
}

// Builds the launch plan (threads per chunk, chunks per workgroup, LDS).
int make_plan(int dtype, int64_t rows, int64_t n, const Geometry& geo, const QSpec* qs, int nq,
              hr::RotPlan* p) {
    memset(p, 0, sizeof *p);
    p->bf16 = dtype == HR_BF16;
    int64_t gmin = INT64_MAX, gmax = 1;
    bool asym_one_group = false;
    for (int i = 0; i < nq; ++i) {
        if (qs[i].g < gmin) gmin = qs[i].g;
        if (qs[i].g > gmax) gmax = qs[i].g;
    }
    // chunk: whole Hadamard blocks and whole groups
    int64_t chunk;
    if (geo.kron_k) {
        chunk = n;
    } else {
        chunk = geo.block;
        if (gmax > chunk) chunk = gmax;
        // small blocks: let one chunk span several blocks so that a thread
        // still owns 16 contiguous elements
        while (chunk < 16 && n % (2 * chunk) == 0) chunk *= 2;
    }
    // elements per thread: at most 16 (32 when a chunk needs it), at most
    // the chunk, and at most the smallest group unless that needs more than
    // 1024 threads
    int64_t e = 16;
    if (chunk / e > 1024) e = 32;
    // one group per thread where that fits 1024 threads; else several whole
    // groups per thread (INT and NVFP4 groups smaller than e)
    if (nq && gmin < e && chunk / gmin <= 1024) e = gmin;
    if (chunk < e) e = chunk;
    if (e < 2) e = 2;
    if (chunk % e) return fail(HR_EUNSUPPORTED, "chunk of %lld elements is not a multiple of %lld",
                                (long long)chunk, (long long)e);
    if (chunk / e > 1024)
        return fail(HR_EUNSUPPORTED, "%lld elements per chunk need more than 1024 threads "
                    "(group_size %lld too small for this block)", (long long)chunk, (long long)gmin);
    if (geo.kron_k && e < 8)
        return fail(HR_EUNSUPPORTED, "Kronecker rotation needs group_size >= 8");
    // several whole groups per thread are quantized by instances for 16 and
    // 32 elements per thread only (groups of 2..8, or 2..16)
    for (int i = 0; i < nq; ++i)
        if (qs[i].g < e && e != 16 && e != 32)
            return fail(HR_EUNSUPPORTED, "group_size %lld is smaller than the %lld elements per thread",
                        (long long)qs[i].g, (long long)e);
    int64_t tpc = chunk / e;
    int64_t cpw = tpc >= 256 ? 1 : 256 / tpc;
    for (int i = 0; i < nq; ++i)
        if (qs[i].format == HR_Q_INT && !qs[i].sym && (cpw * chunk / qs[i].g) % 2) asym_one_group = true;
    // zero points are packed two groups per byte, so a workgroup holds an even
    // number of groups: chunks of one asymmetric group are taken in pairs.
    // Where a pair would need more than 1024 threads, each thread takes 32
    // elements instead of 16 (groups are whole threads: g >= e).
    if (asym_one_group && 2 * cpw * tpc > 1024 && e == 16 && chunk % 32 == 0) {
        e = 32;
        tpc = chunk / e;
        cpw = tpc >= 256 ? 1 : 256 / tpc;
    }
    if (asym_one_group) cpw *= 2;
    const int64_t nt = cpw * tpc;
    if (nt > 1024) return fail(HR_EUNSUPPORTED, "workgroup of %lld threads needed", (long long)nt);
    const int64_t total_elems = rows * n;
    const int64_t total_chunks = total_elems / chunk;
    p->loge = ilog2(e);
    p->nt = static_cast<int>(nt);
    p->grid = (total_chunks + cpw - 1) / cpw;
    if (p->grid > 0x7FFFFFFF) return fail(HR_EUNSUPPORTED, "grid too large");
    if (geo.kron_k)
        p->kmax = geo.kron_k <= 16 ? 16 : (geo.kron_k <= 32 ? 32 : (geo.kron_k <= hr::kMaxKronDense ? 64 : -1));
    const int64_t wg_elems = nt * e;
    size_t lds = static_cast<size_t>(wg_elems + (wg_elems >> 4)) * 4;  // padded transform buffer
    if (p->kmax < 0) lds *= 2;                                          // wide Kronecker mix: output buffer
    lds += static_cast<size_t>(2 * (nt / 64 + 1)) * 4;                  // cross-wave reduction
    // zero-point staging: asymmetric groups at least a thread wide (smaller
    // groups are whole in one thread, which writes their zero points itself)
    int64_t zgroups = 0;
    for (int i = 0; i < nq; ++i)
        if (qs[i].format == HR_Q_INT && !qs[i].sym && qs[i].g >= e && wg_elems / qs[i].g > zgroups)
            zgroups = wg_elems / qs[i].g;
    lds += static_cast<size_t>(zgroups) * 4;
    if (lds > 160 * 1024) return fail(HR_EUNSUPPORTED, "needs %zu bytes of LDS", lds);
    p->lds_bytes = lds;
    hr::RotArgs& a = p->a;
    a.total_chunks = total_chunks;
    a.norm = geo.norm;
    a.logb = geo.logb;
    a.chunk = static_cast<int32_t>(chunk);
    a.tpc = static_cast<int32_t>(tpc);
    a.cpw = static_cast<int32_t>(cpw);
    a.kron_k = geo.kron_k;
    a.nq = nq;
    for (int i = 0; i < nq; ++i) {
        a.total_groups[i] = total_elems / qs[i].g;
        a.q[i].format = qs[i].format;
        a.q[i].sym = qs[i].sym;
        a.q[i].logg = qs[i].logg;
        a.q[i].scale_dtype = qs[i].scale_dtype;
        a.q[i].tscale = qs[i].tscale;
    }
    if (geo.kron_k > hr::kMaxKronDense) {
        if (!hr::paley_character(geo.kron_k, a.kron_chi, hr::kMaxKron / 32))
            return fail(HR_EUNSUPPORTED, "no base matrix of order %d", geo.kron_k);
        a.kron_q = geo.kron_k - 1;
    } else if (geo.kron_k) {
        std::vector<int8_t> h;
        if (!hr::paley_matrix(geo.kron_k, h)) return fail(HR_EUNSUPPORTED, "no base matrix of order %d", geo.kron_k);
        for (int c = 0; c < geo.kron_k; ++c) {
            uint64_t m = 0;
            for (int r = 0; r < geo.kron_k; ++r)
                if (h[static_cast<size_t>(r) * geo.kron_k + c] < 0) m |= uint64_t{1} << r;
            a.hk_neg[c] = m;
        }
    }
    return HR_OK;
}

// Specialised bf16 kernels (one wave per 128 blocks of 32 or 256 of 16, per eight rows of
// 128, or per 4096 elements of blocks of 64 and 256 .. 8192; one workgroup
// per Kronecker row of K x M) take the call when one is compiled for its
// exact shape (randomised rotations: kwave); the generic kernel runs
// otherwise, or always after hr_set_generic_only(1).
// Process-wide dispatch switch (hr_set_generic_only): 1 sends every call to
// the generic kernel, so that tests can run each shape through both paths.
std::atomic<int> g_generic_only{0};

int run(const hr::RotPlan& p, void* stream) {
    if (p.grid == 0) return ok();
    const hr::RotArgs& a = p.a;
    const bool generic_only = g_generic_only.load(std::memory_order_relaxed) != 0;
    const bool mixed = a.perm || a.in_signs || a.out_signs;
    // the specialised kernels read the sign vectors 8 and 16 bytes at a time
    const bool signs_aligned =
        ((reinterpret_cast<uintptr_t>(a.in_signs) | reinterpret_cast<uintptr_t>(a.out_signs)) & 15) == 0;
    // (a chunk is one block, or for blocks smaller than a group several)
    if (!generic_only && p.bf16 && a.kron_k == 0 && signs_aligned &&
        a.logb >= 4 && a.logb <= 13 &&
        a.chunk % (1 << a.logb) == 0) {
        hr::FastKey k{};
        hr::FastArgs f{};
        k.logb = a.logb;
        k.wrot = a.y_rot != nullptr;
        k.mixed = a.perm ? 2 : (mixed ? 1 : 0);
        k.nq = a.nq;
        for (int i = 0; i < a.nq; ++i) {
            k.fmt[i] = a.q[i].format;
            k.sym[i] = a.q[i].sym;
            k.logg[i] = a.q[i].logg;
            k.sdt[i] = a.q[i].scale_dtype;
            f.q[i] = a.q[i];
            f.total_groups[i] = a.total_groups[i];
        }
        f.x = a.x;
        f.y_rot = a.y_rot;
        f.units = a.total_chunks * (a.chunk >> a.logb);   // blocks
        f.norm = a.norm;
        f.perm = a.perm;
        f.in_signs = a.in_signs;
        f.out_signs = a.out_signs;
        f.row_blocks = a.row_n >> a.logb;
        const int r = hr::launch_fast(k, f, stream);
        if (r == 1) return ok();
        if (r < 0)
            return fail(HR_EDEVICE, "kernel launch failed: %s", hipGetErrorString(static_cast<hipError_t>(-r)));
    }
    if (!generic_only && !mixed && p.bf16 && a.nq <= 1 &&
        ((a.kron_k > 0 && a.kron_k <= 32 && a.logb >= 8 && a.logb <= 10) || (a.kron_k > 32 && a.logb == 7))) {
        hr::FastKey k{};
        hr::KronArgs ka{};
        k.logb = a.logb;
        k.wrot = a.y_rot != nullptr;
        k.nq = a.nq;
        if (a.nq == 1) {
            k.fmt[0] = a.q[0].format;
            k.sym[0] = a.q[0].sym;
            k.logg[0] = a.q[0].logg;
            k.sdt[0] = a.q[0].scale_dtype;
            ka.q = a.q[0];
            ka.total_groups = a.total_groups[0];
        }
        ka.x = a.x;
        ka.y_rot = a.y_rot;
        ka.rows = a.total_chunks;
        ka.norm = a.norm;
        ka.k = a.kron_k;
        for (int c = 0; c < a.kron_k && c < hr::kMaxKronDense; ++c) ka.hk_neg[c] = a.hk_neg[c];
        // Sylvester H_M = H_S (x) H_{M/S}, so H_K (x) H_M = (H_K (x) H_S) (x) H_{M/S}:
        // the same row read as S K pieces of M / S.  Small base orders are
        // regrouped this way while S K <= 32 and M / S >= 256, which halves the
        // column blocks the MFMA contracts (and its work per row) at each step.
        // H_K (x) H_S is -1 at (r, c) iff H_K is at (r / S, c / S) xor
        // popcount(r & c & (S - 1)) is odd.
        int sh = 0;
        while (a.kron_k > 0 && (a.kron_k << (sh + 1)) <= 32 && a.logb - (sh + 1) >= 8) ++sh;
        if (sh > 0) {
            ka.k = a.kron_k << sh;
            k.logb = a.logb - sh;
            const int smask = (1 << sh) - 1;
            for (int c = 0; c < ka.k; ++c) {
                uint64_t m = 0;
                for (int r = 0; r < ka.k; ++r) {
                    const uint64_t base = (a.hk_neg[c >> sh] >> (r >> sh)) & 1u;
                    const uint64_t sylv = static_cast<uint64_t>(__builtin_popcount(r & c & smask) & 1);
                    m |= (base ^ sylv) << r;
                }
                ka.hk_neg[c] = m;
            }
        }
        for (int i = 0; i < hr::kMaxKron / 32; ++i) ka.kron_chi[i] = a.kron_chi[i];
        ka.kron_q = a.kron_q;
        const int r = hr::launch_kron(k, ka, stream);
        if (r == 1) return ok();
        if (r < 0)
            return fail(HR_EDEVICE, "kernel launch failed: %s", hipGetErrorString(static_cast<hipError_t>(-r)));
    }
    const int e = hr::launch_rotate(p, stream);
    if (e != 0) return fail(HR_EDEVICE, "kernel launch failed: %s", hipGetErrorString(static_cast<hipError_t>(e)));
    return ok();
}

struct QBuf {
    Range codes, scales, zeros;
};

int check_qbuffers(const QSpec& q, int64_t rows, int64_t n, void* codes, void* scales, void* zeros, const char* tag,
                   QBuf* b) {
    char nm[64];
    snprintf(nm, sizeof nm, "%scodes", tag);
    int st = check_ptr(codes, nm, 16);
    if (st) return st;
    const size_t sal = q.scale_dtype == 0 ? 4 : (q.scale_dtype == 1 ? 2 : 1);
    snprintf(nm, sizeof nm, "%sscales", tag);
    st = check_ptr(scales, nm, sal);
    if (st) return st;
    const int64_t groups = rows * n / q.g;
    b->codes = {"codes", reinterpret_cast<uintptr_t>(codes), reinterpret_cast<uintptr_t>(codes) + (size_t)(rows * n / 2)};
    b->scales = {"scales", reinterpret_cast<uintptr_t>(scales), reinterpret_cast<uintptr_t>(scales) + (size_t)groups * sal};
    b->zeros = {"zeros", 0, 0};
    if (q.format == HR_Q_INT && !q.sym) {
        snprintf(nm, sizeof nm, "%szeros", tag);
        st = check_ptr(zeros, nm, 1);
        if (st) return st;
        b->zeros = {"zeros", reinterpret_cast<uintptr_t>(zeros), reinterpret_cast<uintptr_t>(zeros) + (size_t)((groups + 1) / 2)};
    } else if (zeros) {
        return fail(HR_EINVAL, "%szeros must be NULL for a symmetric, MXFP4 or NVFP4 quantizer", tag);
    }
    return HR_OK;
}

int check_disjoint(const std::vector<Range>& rs) {
    for (size_t i = 0; i < rs.size(); ++i)
        for (size_t j = i + 1; j < rs.size(); ++j)
            if (rs[i].hi > rs[i].lo && rs[j].hi > rs[j].lo && overlap(rs[i], rs[j]))
                return fail(HR_EINVAL, "buffers %s and %s overlap", rs[i].name, rs[j].name);
    return HR_OK;
}

// Validated randomised-rotation vectors; ranges for the overlap checks.
struct Mix {
    const int32_t* perm = nullptr;
    const int8_t* in_signs = nullptr;
    const int8_t* out_signs = nullptr;
    std::vector<Range> ranges;
    bool any() const { return perm || in_signs || out_signs; }
};

int check_mix(const hr_mix* m, int64_t n, Mix* out) {
    *out = Mix{};
    if (!m) return HR_OK;
    if ((m->perm || m->in_signs || m->out_signs) && n > INT32_MAX)
        return fail(HR_EINVAL, "n = %lld: a randomised rotation needs n < 2^31", (long long)n);
    out->perm = m->perm;
    out->in_signs = m->in_signs;
    out->out_signs = m->out_signs;
    if (m->perm) {
        int st = check_ptr(m->perm, "mix->perm", 4);
        if (st) return st;
        out->ranges.push_back({"mix->perm", reinterpret_cast<uintptr_t>(m->perm),
                               reinterpret_cast<uintptr_t>(m->perm) + static_cast<size_t>(n) * 4});
    }
    if (m->in_signs)
        out->ranges.push_back({"mix->in_signs", reinterpret_cast<uintptr_t>(m->in_signs),
                               reinterpret_cast<uintptr_t>(m->in_signs) + static_cast<size_t>(n)});
    if (m->out_signs)
        out->ranges.push_back({"mix->out_signs", reinterpret_cast<uintptr_t>(m->out_signs),
                               reinterpret_cast<uintptr_t>(m->out_signs) + static_cast<size_t>(n)});
    return HR_OK;
}

// The mix vectors are inputs: no output may overlap them.
int check_mix_outputs(const Mix& mx, const std::vector<Range>& outs) {
    for (const Range& m : mx.ranges)
        for (const Range& o : outs)
            if (o.hi > o.lo && overlap(m, o)) return fail(HR_EINVAL, "output %s overlaps %s", o.name, m.name);
    return HR_OK;
}

void apply_mix(const Mix& mx, int64_t n, hr::RotPlan* p) {
    p->a.perm = mx.perm;
    p->a.in_signs = mx.in_signs;
    p->a.out_signs = mx.out_signs;
    p->a.row_n = n;
}

int rotate_impl(const void* x, void* y, int dtype, int64_t rows, int64_t n, int64_t block, const hr_mix* mix,
                void* stream) {
    int st = check_shape(dtype, rows, n);
    if (st) return st;
    Geometry geo;
    st = check_block(n, block, &geo);
    if (st) return st;
    Mix mx;
    if ((st = check_mix(mix, n, &mx))) return st;
    if (rows == 0) return ok();
    if ((st = check_ptr(x, "x", 16)) || (st = check_ptr(y, "y", 16))) return st;
    const size_t bytes = static_cast<size_t>(rows * n) * dtype_size(dtype);
    Range ry{"y", reinterpret_cast<uintptr_t>(y), reinterpret_cast<uintptr_t>(y) + bytes};
    if (x != y) {
        Range rx{"x", reinterpret_cast<uintptr_t>(x), reinterpret_cast<uintptr_t>(x) + bytes};
        if (overlap(rx, ry)) return fail(HR_EINVAL, "y partially overlaps x");
    } else if (mx.perm) {
        return fail(HR_EINVAL, "a permuted rotation cannot run in place (y == x)");
    }
    if ((st = check_mix_outputs(mx, {ry}))) return st;
    hr::RotPlan p;
    st = make_plan(dtype, rows, n, geo, nullptr, 0, &p);
    if (st) return st;
    p.a.x = x;
    p.a.y_rot = y;
    apply_mix(mx, n, &p);
    return run(p, stream);
}

int act_impl(const void* x, int dtype, int64_t rows, int64_t n, int64_t block, const hr_qspec* q, void* codes,
             void* scales, void* zeros, void* y_rot, const hr_mix* mix, void* stream) {
    int st = check_shape(dtype, rows, n);
    if (st) return st;
    Geometry geo;
    if ((st = check_block(n, block, &geo))) return st;
    QSpec qs;
    if ((st = check_qspec(q, n, &qs))) return st;
    Mix mx;
    if ((st = check_mix(mix, n, &mx))) return st;
    if (rows == 0) return ok();
    if ((st = check_ptr(x, "x", 16))) return st;
    QBuf b;
    if ((st = check_qbuffers(qs, rows, n, codes, scales, zeros, "", &b))) return st;
    const size_t bytes = static_cast<size_t>(rows * n) * dtype_size(dtype);
    Range rx{"x", reinterpret_cast<uintptr_t>(x), reinterpret_cast<uintptr_t>(x) + bytes};
    std::vector<Range> rs{b.codes, b.scales, b.zeros};
    if (y_rot) {
        if ((st = check_ptr(y_rot, "y_rot", 16))) return st;
        Range ry{"y_rot", reinterpret_cast<uintptr_t>(y_rot), reinterpret_cast<uintptr_t>(y_rot) + bytes};
        if (y_rot != x && overlap(rx, ry)) return fail(HR_EINVAL, "y_rot partially overlaps x");
        if (y_rot == x && mx.perm) return fail(HR_EINVAL, "a permuted rotation cannot run in place (y_rot == x)");
        rs.push_back(ry);
    }
    if ((st = check_disjoint(rs))) return st;
    for (const Range& r : std::vector<Range>{b.codes, b.scales, b.zeros})
        if (r.hi > r.lo && overlap(r, rx)) return fail(HR_EINVAL, "output %s overlaps x", r.name);
    if ((st = check_mix_outputs(mx, rs))) return st;
    hr::RotPlan p;
    if ((st = make_plan(dtype, rows, n, geo, &qs, 1, &p))) return st;
    p.a.x = x;
    p.a.y_rot = y_rot;
    p.a.q[0].codes = static_cast<uint8_t*>(codes);
    p.a.q[0].scales = scales;
    p.a.q[0].zeros = static_cast<uint8_t*>(zeros);
    apply_mix(mx, n, &p);
    return run(p, stream);
}

int weight_impl(const void* w, int dtype, int64_t out_features, int64_t in_features, int64_t block, void* w_rot,
                const hr_qspec* q, int nq, const hr_qout* outs, const hr_mix* mix, void* stream) {
    const int64_t rows = out_features, n = in_features;
    int st = check_shape(dtype, rows, n);
    if (st) return st;
    Geometry geo;
    if ((st = check_block(n, block, &geo))) return st;
    if (nq < 0 || nq > hr::kMaxQuant) return fail(HR_EINVAL, "nq = %d must be 0, 1 or 2", nq);
    if (nq > 0 && (!q || !outs)) return fail(HR_EINVAL, "q and outs must be given when nq > 0");
    if (nq == 0 && !w_rot) return fail(HR_EINVAL, "nothing to compute: w_rot is NULL and nq = 0");
    QSpec qs[hr::kMaxQuant];
    for (int i = 0; i < nq; ++i)
        if ((st = check_qspec(&q[i], n, &qs[i]))) return st;
    Mix mx;
    if ((st = check_mix(mix, n, &mx))) return st;
    if (rows == 0) return ok();
    if ((st = check_ptr(w, "w", 16))) return st;
    const size_t bytes = static_cast<size_t>(rows * n) * dtype_size(dtype);
    Range rw{"w", reinterpret_cast<uintptr_t>(w), reinterpret_cast<uintptr_t>(w) + bytes};
    std::vector<Range> rs;
    if (w_rot) {
        if ((st = check_ptr(w_rot, "w_rot", 16))) return st;
        rs.push_back({"w_rot", reinterpret_cast<uintptr_t>(w_rot), reinterpret_cast<uintptr_t>(w_rot) + bytes});
    }
    for (int i = 0; i < nq; ++i) {
        QBuf b;
        const char* tag = i == 0 ? "outs[0]." : "outs[1].";
        if ((st = check_qbuffers(qs[i], rows, n, outs[i].codes, outs[i].scales, outs[i].zeros, tag, &b))) return st;
        rs.push_back(b.codes);
        rs.push_back(b.scales);
        rs.push_back(b.zeros);
    }
    if ((st = check_disjoint(rs))) return st;
    for (const Range& r : rs)
        if (r.hi > r.lo && overlap(r, rw)) return fail(HR_EINVAL, "output %s overlaps w", r.name);
    if ((st = check_mix_outputs(mx, rs))) return st;
    hr::RotPlan p;
    if ((st = make_plan(dtype, rows, n, geo, qs, nq, &p))) return st;
    p.a.x = w;
    p.a.y_rot = w_rot;
    for (int i = 0; i < nq; ++i) {
        p.a.q[i].codes = static_cast<uint8_t*>(outs[i].codes);
        p.a.q[i].scales = outs[i].scales;
        p.a.q[i].zeros = static_cast<uint8_t*>(outs[i].zeros);
    }
    apply_mix(mx, n, &p);
    return run(p, stream);
}

// dequant_check and dequant_check_noalloc: the statistics partials go to
// the caller's `work` or, with use_static, to the library's static device
// scratch (no allocation either way).
int dequant_impl(const void* codes, const void* scales, const void* zeros, const hr_qspec* q, int64_t rows,
                 int64_t n, const void* ref, int ref_dtype, float* deq, hr_dq_stats* stats, void* work,
                 bool use_static, void* stream) {
    static_assert(hr::kDqWorkBytes <= HR_DQ_WORK_BYTES, "dequant_check workspace");
    int st = check_shape(HR_F32, rows, n);
    if (st) return st;
    QSpec qs;
    if ((st = check_qspec(q, n, &qs))) return st;
    if (!deq && !stats) return fail(HR_EINVAL, "nothing to compute: deq and stats are NULL");
    if (stats && !ref) return fail(HR_EINVAL, "stats requires ref");
    if (stats && !work && !use_static)
        return fail(HR_EINVAL, "stats requires work (HR_DQ_WORK_BYTES of device memory)");
    if (ref && ref_dtype != HR_F32 && ref_dtype != HR_BF16) return fail(HR_EINVAL, "ref_dtype must be HR_F32 or HR_BF16");
    if (rows == 0) {
        if (stats) memset(stats, 0, sizeof *stats);
        return ok();
    }
    QBuf b;
    if ((st = check_qbuffers(qs, rows, n, const_cast<void*>(codes), const_cast<void*>(scales),
                             const_cast<void*>(zeros), "", &b)))
        return st;
    std::vector<Range> ins{b.codes, b.scales, b.zeros};
    if (ref) {
        if ((st = check_ptr(ref, "ref", 16))) return st;
        ins.push_back({"ref", reinterpret_cast<uintptr_t>(ref),
                       reinterpret_cast<uintptr_t>(ref) + (size_t)(rows * n) * dtype_size(ref_dtype)});
    }
    std::vector<Range> outs;
    if (deq) {
        if ((st = check_ptr(deq, "deq", 16))) return st;
        outs.push_back({"deq", reinterpret_cast<uintptr_t>(deq), reinterpret_cast<uintptr_t>(deq) + (size_t)(rows * n) * 4});
    }
    if (stats && !use_static) {
        if ((st = check_ptr(work, "work", 16))) return st;
        outs.push_back({"work", reinterpret_cast<uintptr_t>(work), reinterpret_cast<uintptr_t>(work) + HR_DQ_WORK_BYTES});
    }
    for (const Range& o : outs)
        for (const Range& r : ins)
            if (r.hi > r.lo && overlap(r, o)) return fail(HR_EINVAL, "%s overlaps %s", o.name, r.name);
    if ((st = check_disjoint(outs))) return st;
    if (stats && use_static) {
        // one call's partials: at most kDqMaxParts + 1 slots whatever the
        // input size (the grid is capped and strides over the rest), which
        // the static scratch holds (checked at compile time)
        const int e = hr::scratch_address(&work);
        if (e != 0)
            return fail(HR_EDEVICE, "static scratch unavailable: %s", hipGetErrorString(static_cast<hipError_t>(e)));
    }
    hr::DqArgs a{};
    a.codes = static_cast<const uint8_t*>(codes);
    a.scales = scales;
    a.zeros = static_cast<const uint8_t*>(zeros);
    a.ref = stats ? ref : nullptr;
    a.deq = deq;
    a.parts = stats ? work : nullptr;
    a.total = rows * n;
    a.format = qs.format;
    a.sym = qs.sym;
    a.logg = qs.logg;
    a.scale_dtype = qs.scale_dtype;
    a.tscale = qs.tscale;
    a.ref_bf16 = ref_dtype == HR_BF16;
    const int le = hr::launch_dequant(a, stream);
    if (le != 0) return fail(HR_EDEVICE, "kernel launch failed: %s", hipGetErrorString(static_cast<hipError_t>(le)));
    if (stats) {
        hipStream_t s = static_cast<hipStream_t>(stream);
        hr::DqPartial h;
        hipError_t e = hipMemcpyAsync(&h, static_cast<const hr::DqPartial*>(work) + hr::kDqMaxParts, sizeof h,
                                      hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return fail(HR_EDEVICE, "reading statistics failed: %s", hipGetErrorString(e));
        stats->max_err_steps = h.max_err;
        stats->n_over_half_step = static_cast<int64_t>(h.n_over);
        stats->n_clamped = static_cast<int64_t>(h.n_clamped);
        stats->rel_l2_err = h.sum_ref2 > 0 ? sqrt(h.sum_err2 / h.sum_ref2) : 0.0;
    }
    return ok();
}

}  // namespace

extern "C" {

const char* hr_last_error(void) { return g_err.c_str(); }

int hr_kron_order(int64_t n, int32_t* K, int64_t* M, int8_t* hk) {
    if (n <= 0 || is_pow2(n)) return fail(HR_EINVAL, "n = %lld is not a positive non-power-of-two", (long long)n);
    const int64_t k = hr::kron_order(n);
    if (k == 0) return fail(HR_EUNSUPPORTED, "no supported base Hadamard order for n = %lld", (long long)n);
    if (K) *K = static_cast<int32_t>(k);
    if (M) *M = n / k;
    if (hk) {
        std::vector<int8_t> h;
        if (!hr::paley_matrix(static_cast<int>(k), h)) return fail(HR_EUNSUPPORTED, "no base matrix");
        memcpy(hk, h.data(), h.size());
    }
    return ok();
}

int hadamard_rotate(const void* x, void* y, int dtype, int64_t rows, int64_t n, int64_t block, void* stream) {
    return rotate_impl(x, y, dtype, rows, n, block, nullptr, stream);
}

int hadamard_rotate_mixed(const void* x, void* y, int dtype, int64_t rows, int64_t n, int64_t block,
                          const hr_mix* mix, void* stream) {
    return rotate_impl(x, y, dtype, rows, n, block, mix, stream);
}

int rotate_quantize_act(const void* x, int dtype, int64_t rows, int64_t n, int64_t block, const hr_qspec* q,
                        void* codes, void* scales, void* zeros, void* y_rot, void* stream) {
    return act_impl(x, dtype, rows, n, block, q, codes, scales, zeros, y_rot, nullptr, stream);
}

int rotate_quantize_act_mixed(const void* x, int dtype, int64_t rows, int64_t n, int64_t block, const hr_qspec* q,
                              void* codes, void* scales, void* zeros, void* y_rot, const hr_mix* mix, void* stream) {
    return act_impl(x, dtype, rows, n, block, q, codes, scales, zeros, y_rot, mix, stream);
}

int rotate_fuse_weight(const void* w, int dtype, int64_t out_features, int64_t in_features, int64_t block,
                       void* w_rot, const hr_qspec* q, int nq, const hr_qout* outs, void* stream) {
    return weight_impl(w, dtype, out_features, in_features, block, w_rot, q, nq, outs, nullptr, stream);
}

int rotate_fuse_weight_mixed(const void* w, int dtype, int64_t out_features, int64_t in_features, int64_t block,
                             void* w_rot, const hr_qspec* q, int nq, const hr_qout* outs, const hr_mix* mix,
                             void* stream) {
    return weight_impl(w, dtype, out_features, in_features, block, w_rot, q, nq, outs, mix, stream);
}

int rotate_fuse_weight_out(const void* w, int dtype, int64_t out_features, int64_t in_features, int64_t block,
                           void* w_rot, void* stream) {
    int st = check_shape(dtype, out_features, in_features);
    if (st) return st;
    if (out_features == 0) return ok();
    const int64_t b = (block <= 0 || block == out_features) ? out_features : block;
    if (block > 0 && !is_pow2(block))
        return fail(HR_EINVAL, "block = %lld is not a power of two", (long long)block);
    if (out_features % b)
        return fail(HR_EINVAL, "block %lld does not divide out_features = %lld", (long long)b, (long long)out_features);
    hr::ColArgs a{};
    if (is_pow2(b) && b >= 32 && b <= 4096) {
        // colrot: tiles of b rows x C columns
        const int logb = ilog2(b);
        // tile of b rows x C columns: C >= 8, b C = 2^14 where that allows (or
        // the largest power of two below it that divides in_features, down to
        // 2^11 elements)
        constexpr int kColTileLog = 14;
        int64_t C = int64_t{1} << (logb + 3 > kColTileLog ? 3 : kColTileLog - logb);
        while (C > 8 && in_features % C) C >>= 1;
        if (in_features % C || b * C < 2048)
            return fail(HR_EUNSUPPORTED, "in_features = %lld must be a multiple of %lld for blocks of %lld rows",
                        (long long)in_features, (long long)(2048 / b > 8 ? 2048 / b : 8), (long long)b);
        if ((out_features / b) * (in_features / C) >= (int64_t{1} << 31))
            return fail(HR_EINVAL, "tensor too large (out_features = %lld, in_features = %lld)", (long long)out_features,
                        (long long)in_features);
        a.logb = logb;
        a.strips = in_features / C;
        a.tb = ilog2(b * C);
    } else {
        // colwide: tiles of all b = K M rows x 4 columns (a Sylvester block of
        // 8192 rows, or the Kronecker form of a full-width b that is not a
        // power of two)
        int64_t K = 1, M = b;
        if (!is_pow2(b)) {
            if (block > 0) return fail(HR_EINVAL, "block = %lld is not a power of two", (long long)block);
            K = hr::kron_order(b);
            if (K == 0)
                return fail(HR_EUNSUPPORTED, "no supported base Hadamard order for out_features = %lld", (long long)b);
            M = b / K;
        }
        const bool shape_ok = (K == 1 && b == 8192) ||
                              ((K == 12 || K == 20 || K == 28) && b <= 8192 && b % 512 == 0 && M >= 128);
        if (!shape_ok)
            return fail(HR_EUNSUPPORTED,
                        "output-side rotation of %lld rows: blocks of 32..4096 or 8192 rows, or K x M rows with K "
                        "12, 20 or 28, K M a multiple of 512 and at most 8192 (got K = %lld, M = %lld)",
                        (long long)b, (long long)K, (long long)M);
        if (in_features % 4)
            return fail(HR_EUNSUPPORTED, "in_features = %lld must be a multiple of 4 for %lld rows",
                        (long long)in_features, (long long)b);
        if ((out_features / b) * (in_features / 4) >= (int64_t{1} << 31))
            return fail(HR_EINVAL, "tensor too large (out_features = %lld, in_features = %lld)", (long long)out_features,
                        (long long)in_features);
        a.logb = ilog2(M);
        a.strips = in_features / 4;
        a.kron_k = static_cast<int32_t>(K);
        if (K > 1) {
            std::vector<int8_t> h;
            if (!hr::paley_matrix(static_cast<int>(K), h)) return fail(HR_EUNSUPPORTED, "no base matrix of order %lld", (long long)K);
            for (int o = 0; o < K; ++o) {
                uint64_t m = 0;
                for (int c = 0; c < K; ++c)
                    if (h[static_cast<size_t>(c) * K + o] < 0) m |= uint64_t{1} << c;
                a.hk_neg[o] = m;
            }
        }
    }
    if ((st = check_ptr(w, "w", 16)) || (st = check_ptr(w_rot, "w_rot", 16))) return st;
    const size_t bytes = static_cast<size_t>(out_features * in_features) * dtype_size(dtype);
    if (w != w_rot) {
        Range rw{"w", reinterpret_cast<uintptr_t>(w), reinterpret_cast<uintptr_t>(w) + bytes};
        Range ry{"w_rot", reinterpret_cast<uintptr_t>(w_rot), reinterpret_cast<uintptr_t>(w_rot) + bytes};
        if (overlap(rw, ry)) return fail(HR_EINVAL, "w_rot partially overlaps w");
    }
    a.w = w;
    a.w_rot = w_rot;
    a.in = in_features;
    a.row_blocks = out_features / b;
    a.norm = static_cast<float>(1.0 / sqrt(static_cast<double>(b)));
    a.bf16 = dtype == HR_BF16;
    const int e = hr::launch_colrot(a, stream);
    if (e != 0) return fail(HR_EDEVICE, "kernel launch failed: %s", hipGetErrorString(static_cast<hipError_t>(e)));
    return ok();
}

int dequant_check(const void* codes, const void* scales, const void* zeros, const hr_qspec* q, int64_t rows,
                  int64_t n, const void* ref, int ref_dtype, float* deq, hr_dq_stats* stats, void* work,
                  void* stream) {
    return dequant_impl(codes, scales, zeros, q, rows, n, ref, ref_dtype, deq, stats, work, false, stream);
}

int dequant_check_noalloc(const void* codes, const void* scales, const void* zeros, const hr_qspec* q, int64_t rows,
                          int64_t n, const void* ref, int ref_dtype, float* deq, hr_dq_stats* stats, void* stream) {
    return dequant_impl(codes, scales, zeros, q, rows, n, ref, ref_dtype, deq, stats, nullptr, true, stream);
}

void hr_set_generic_only(int on) { g_generic_only.store(on ? 1 : 0, std::memory_order_relaxed); }

int hr_check_shape(int dtype, int64_t rows, int64_t n, int64_t block, const hr_qspec* q, int nq) {
    int st = check_shape(dtype, rows, n);
    if (st) return st;
    Geometry geo;
    if ((st = check_block(n, block, &geo))) return st;
    if (nq < 0 || nq > hr::kMaxQuant) return fail(HR_EINVAL, "nq = %d must be 0, 1 or 2", nq);
    if (nq > 0 && !q) return fail(HR_EINVAL, "q must be given when nq > 0");
    QSpec qs[hr::kMaxQuant];
    for (int i = 0; i < nq; ++i)
        if ((st = check_qspec(&q[i], n, &qs[i]))) return st;
    hr::RotPlan p;
    if ((st = make_plan(dtype, rows > 0 ? rows : 1, n, geo, qs, nq, &p))) return st;
    return ok();
}

}  // extern "C"
