// C ABI of libmambascan: argument validation, launch planning and dispatch.
// Declarations and the contract live in include/mamba_scan.h.
#include "mamba_scan.h"

#include "relay.h"
#include "scan_common.h"
#include "scan_bwd.h"
#include "ssd.h"

#include <algorithm>
#include <limits.h>
#include <stdint.h>

using namespace mambascan;

namespace {

// Kernel family used when the caller does not choose one: the scalar-B/C kernel for
// d_state up to 32 (with or without a sequence split: measured fastest or equal on the
// small prefill and the long sequence, 104 us against 108 us and 1.71 ms against 1.82 ms
// at the best span count of each); d_state 64, which it does not compile, uses the
// barrier-free row kernel.
Family auto_family(int64_t batch, int64_t d_inner, int64_t d_state, int cus)
{
    (void)batch;
    (void)d_inner;
    (void)cus;
    return d_state <= 32 ? Family::Scalar : Family::Rows;
}

// Scalar-family defaults: (waves, chunk) = (4, 8), (8, 8), (8, 8), (8, 4) for d_state 4..32.
int scalar_default_waves(int64_t d_state) { return d_state >= 8 ? 8 : 4; }
int scalar_default_chunk(int64_t d_state) { return d_state == 32 ? 4 : 8; }

// The scalar kernel addresses one span of one batch row of an activation tensor with
// 32-bit byte offsets: span length x d_inner x 4 bytes (fp32, the larger element) must
// stay below 2^31.
bool scalar_span_ok(int64_t span_len, int64_t d_inner)
{
    return d_inner <= INT32_MAX / 4 && span_len <= (int64_t)(INT32_MAX / 4) / d_inner;
}

struct Range {
    uintptr_t lo, hi; // [lo, hi)
};

Range range_of(const void *p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, p && bytes > 0 ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlaps(Range a, Range b)
{
    if (a.hi == a.lo || b.hi == b.lo)
        return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }

// d_state values the scan kernels are compiled for; any other d_state in 1..64 runs at the
// next compiled size with the state arrays padded (pad.hip), padded_d_state giving that size
// (0: not supported).
bool d_state_ok(int64_t n) { return n == 4 || n == 8 || n == 16 || n == 32 || n == 64; }
bool bwd_d_state_ok(int64_t n) { return n == 4 || n == 8 || n == 16 || n == 32; }
int64_t padded_d_state(int64_t n)
{
    if (n < 1 || n > 64)
        return 0;
    int64_t p = 4;
    while (p < n)
        p *= 2;
    return p;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Row strides of the activations, in elements (mamba_scan_ext_t; 0 = contiguous).
struct Rows {
    int64_t u, d, z, B, C;
    bool strided;   // some stride is not its row length: the scalar family reads those
    int64_t widest; // the largest of u, d, z and d_inner (the scalar kernel's span bytes)
};

// false if a stride is negative or shorter than its row
bool rows_of(const mamba_scan_ext_t *ext, int64_t d_inner, int64_t d_state, Rows *r)
{
    auto one = [](int64_t s, int64_t row, int64_t *out) {
        *out = s == 0 ? row : s;
        return s == 0 || s >= row;
    };
    const bool ok = one(ext ? ext->u_stride : 0, d_inner, &r->u) &&
                    one(ext ? ext->delta_stride : 0, d_inner, &r->d) &&
                    one(ext ? ext->z_stride : 0, d_inner, &r->z) &&
                    one(ext ? ext->B_stride : 0, d_state, &r->B) &&
                    one(ext ? ext->C_stride : 0, d_state, &r->C);
    r->strided = r->u != d_inner || r->d != d_inner || r->z != d_inner || r->B != d_state ||
                 r->C != d_state;
    r->widest = std::max(std::max(r->u, r->d), std::max(r->z, d_inner));
    return ok;
}

// Bytes from the first element of `rows` rows of `row` elements, `stride` apart, to the
// end of the last one; -1 on overflow.
int64_t extent_bytes(int64_t rows, int64_t stride, int64_t row, int64_t es)
{
    int64_t t;
    if (rows <= 0 || row <= 0)
        return 0;
    if (!mul_ok(rows - 1, stride, &t) || t > INT64_MAX - row || !mul_ok(t + row, es, &t))
        return -1;
    return t;
}

// Workspace prefix of a padded forward call: the padded copies of A, B, C, h0, theta,
// B_prev and the padded final state, each 256-byte aligned (h0 and the final state always
// reserved: the size query does not know whether they are given).
struct FwdPad {
    size_t a, b, c, h0, hl, theta, bprev, total;
};

bool fwd_pad_layout(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t np, int64_t es,
                    bool theta, bool bprev, FwdPad *f)
{
    int64_t a, bl, bd, t;
    if (!mul_ok(d_inner, np * 4, &a) || !mul_ok(batch, seqlen, &t) || !mul_ok(t, np * es, &bl) ||
        !mul_ok(batch, d_inner, &t) || !mul_ok(t, np * 4, &bd))
        return false;
    size_t o = 0;
    f->a = o;
    o += align256((size_t)a);
    f->b = o;
    o += align256((size_t)bl);
    f->c = o;
    o += align256((size_t)bl);
    f->h0 = o;
    o += align256((size_t)bd);
    f->hl = o;
    o += align256((size_t)bd);
    f->theta = o;
    if (theta)
        o += align256((size_t)bl / 2);
    f->bprev = o;
    if (bprev)
        o += align256((size_t)(batch * np * es));
    f->total = o;
    return true;
}

// Workspace prefix of a padded backward call: the padded copies of A, B, C, h0, dh_last
// and the padded gradients dB, dC, dA, dh0 (B/C-shaped slots sized for 4-byte elements:
// the size query does not know the dtype).
struct BwdPad {
    size_t a, b, c, h0, dhl, db, dc, da, dh0, total;
};

bool bwd_pad_layout(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t np, BwdPad *f)
{
    int64_t a, bl, bd, t;
    if (!mul_ok(d_inner, np * 4, &a) || !mul_ok(batch, seqlen, &t) || !mul_ok(t, np * 4, &bl) ||
        !mul_ok(batch, d_inner, &t) || !mul_ok(t, np * 4, &bd))
        return false;
    size_t o = 0;
    auto put = [&](size_t *slot, int64_t bytes) {
        *slot = o;
        o += align256((size_t)bytes);
    };
    put(&f->a, a);
    put(&f->b, bl);
    put(&f->c, bl);
    put(&f->h0, bd);
    put(&f->dhl, bd);
    put(&f->db, bl);
    put(&f->dc, bl);
    put(&f->da, a);
    put(&f->dh0, bd);
    f->total = o;
    return true;
}

// Bytes of the backward-pass checkpoints: (batch * channel tiles) x ceil(L / 8) segments x
// d_state x 64 lanes, fp32; -1 on overflow.
int64_t ckpt_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state)
{
    int64_t t;
    const int64_t units = batch * ((d_inner + 63) / 64), nseg = (seqlen + 7) / 8;
    if (!mul_ok(units, nseg, &t) || !mul_ok(t, d_state * 64 * 4, &t))
        return -1;
    return t;
}

int cu_count()
{
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cu <= 0) {
        (void)hipGetLastError(); // do not leave a sticky error behind
        return 256;
    }
    return cu;
}

struct Plan {
    Family family;
    int waves, chunk, n_spans;
    int64_t span_len;
    int relay_parts;      // 1: no relay
    int64_t relay_tiles;  // relayed (batch row, tile) units
    int64_t relay_len;    // steps per relay part (a multiple of chunk)
    bool relay_withhold;  // failure test: part 0 withholds its hand-off (relay = -k)
    bool zoh;             // zero-order-hold discretisation (scalar family only)
    bool trap, rot;       // exponential-trapezoidal input term, pair rotation (scalar family)
    bool ckpt;            // backward-pass checkpoints written (scalar family, Euler)
};

// Launch plan.  Channel tiles of 64 lanes x `waves` waves are the unit of parallel work;
// when a single span cannot give every SIMD a few waves, the sequence is split into spans
// (at most 64, each at least 256 steps) joined by the carry pass.
mamba_status_t make_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                         const mamba_scan_opts_t *opts, const mamba_scan_ext_t *ext, Plan *plan,
                         const Rows *rows)
{
    Plan p{};
    const bool strided = rows && rows->strided;
    const int64_t widest = rows ? rows->widest : d_inner;
    const int cus = cu_count();
    const int fam = opts ? opts->kernel : MAMBA_KERNEL_AUTO;
    const int disc = opts ? opts->discretization : MAMBA_DISC_EULER;
    if (disc != MAMBA_DISC_EULER && disc != MAMBA_DISC_ZOH)
        return MAMBA_ERR_UNSUPPORTED;
    p.zoh = disc == MAMBA_DISC_ZOH;
    p.trap = ext && ext->lambda;
    p.rot = ext && ext->theta;
    p.ckpt = ext && ext->ckpt;
    if (p.trap && p.zoh)
        return MAMBA_ERR_UNSUPPORTED; // the trapezoid replaces the input term
    if (p.ckpt && (p.zoh || p.trap || p.rot || !bwd_d_state_ok(d_state)))
        return MAMBA_ERR_UNSUPPORTED; // the backward pass is built for Euler only
    Family autof = auto_family(batch, d_inner, d_state, cus);
    if (autof == Family::Scalar && !scalar_span_ok(seqlen, widest))
        autof = Family::Rows;
    if (p.zoh || p.trap || p.rot || p.ckpt || strided) {
        // these options (and strided rows) are implemented in the scalar-B/C family only
        if (fam == MAMBA_KERNEL_ROWS || fam == MAMBA_KERNEL_BLOCK)
            return MAMBA_ERR_UNSUPPORTED;
        autof = Family::Scalar;
    }
    if (fam == MAMBA_KERNEL_AUTO && opts && (opts->waves || opts->chunk_len)) {
        // an explicit block shape: the scalar family if it has it, else the block family
        const int w = opts->waves ? opts->waves : scalar_default_waves(d_state);
        const int c = opts->chunk_len ? opts->chunk_len : scalar_default_chunk(d_state);
        autof = scalar_variant_supported(d_state, w, c) || p.zoh || p.trap || p.rot ||
                        p.ckpt || strided
                    ? Family::Scalar : Family::Block;
    }
    if (fam == MAMBA_KERNEL_ROWS || (fam == MAMBA_KERNEL_AUTO && autof == Family::Rows)) {
        if ((opts && (opts->waves || opts->chunk_len)))
            return MAMBA_ERR_UNSUPPORTED; // fixed shape: 4 waves x 16 channels, 4-step blocks
        p.family = Family::Rows;
        p.waves = 4;
        p.chunk = 4;
    } else if (fam == MAMBA_KERNEL_SCALAR ||
               (fam == MAMBA_KERNEL_AUTO && autof == Family::Scalar)) {
        p.family = Family::Scalar;
        p.waves = opts && opts->waves ? opts->waves : scalar_default_waves(d_state);
        p.chunk = opts && opts->chunk_len ? opts->chunk_len : scalar_default_chunk(d_state);
        if (!scalar_variant_supported(d_state, p.waves, p.chunk))
            return MAMBA_ERR_UNSUPPORTED;
    } else if (fam == MAMBA_KERNEL_BLOCK || (fam == MAMBA_KERNEL_AUTO && autof == Family::Block)) {
        p.family = Family::Block;
        p.waves = opts && opts->waves ? opts->waves : default_waves(d_state);
        p.chunk = opts && opts->chunk_len ? opts->chunk_len : default_chunk(d_state, p.waves);
        if (!scan_variant_supported(d_state, p.waves, p.chunk))
            return MAMBA_ERR_UNSUPPORTED;
    } else {
        return MAMBA_ERR_UNSUPPORTED;
    }
    // the rotation turns state pairs (2k, 2k+1), which must sit in one wave (its span
    // summaries are the pairs' 2x2 transitions)
    if (p.rot && (d_state % 2 != 0 || (d_state / p.waves) % 2 != 0))
        return MAMBA_ERR_UNSUPPORTED;
    const bool fixed_spans = opts && opts->n_spans;
    int spans = 1;
    if (fixed_spans) {
        if (opts->n_spans < 1 || opts->n_spans > 64)
            return MAMBA_ERR_UNSUPPORTED;
        spans = opts->n_spans;
    } else {
        const int64_t tiles = batch * ((d_inner + 63) / 64);
        const int64_t waves_per_span = tiles * p.waves;
        const int64_t want = (int64_t)cus * 4 /*SIMDs*/ * 4 /*waves each*/;
        if (waves_per_span * 2 < want) {
            // A split sequence runs the END pass over (S - 1) / S of it whatever S is, so
            // once split, spans are cheap: the scalar kernel takes enough for ~12 waves per
            // SIMD (span-count sweep: long sequence 2.13 / 1.87 / 1.71 ms at 16 / 32 / 64
            // spans; small prefill 139 / 104 / 107 us at 4 / 8 / 16, capped there by the
            // 256-step minimum span), the row kernel enough for 4.
            const int64_t target = p.family == Family::Scalar ? want * 3 : want;
            int64_t s = 1;
            while (s * waves_per_span < target && s < 64)
                s <<= 1;
            const int64_t by_len = seqlen / 256;
            if (s > by_len)
                s = by_len > 1 ? by_len : 1;
            spans = (int)s;
        }
    }
    if (seqlen <= 0)
        spans = 1;
    int64_t len = 0;
    for (;;) {
        // span length: a multiple of the chunk so that only the last span has a partial chunk
        len = (seqlen + spans - 1) / spans;
        len = (len + p.chunk - 1) / p.chunk * p.chunk;
        if (len < p.chunk)
            len = p.chunk;
        if (p.family != Family::Scalar || scalar_span_ok(len, widest))
            break;
        if (fixed_spans || spans >= 64)
            return MAMBA_ERR_UNSUPPORTED; // span too large for the scalar kernel's addressing
        spans *= 2;
    }
    spans = (int)((seqlen + len - 1) / len);
    if (spans < 1)
        spans = 1;
    p.n_spans = spans;
    p.span_len = len;

    // Relay: with U units over `cus` compute units, U mod cus units would make a last,
    // mostly idle round.  Splitting each of them in time into two halves, the first run in
    // the first round and the second in the last round (workgroups are dispatched in index
    // order, round-robin over compute units), gives those compute units half a unit each
    // instead of a whole one (measured at 8 x 4096 x 5120: 747 us against 816 us; a 5/8
    // first part gave 784 us).  More than two parts would chain inside the last round.
    // Forced part counts (testing) use equal parts; a negative count -k forces k parts whose
    // first part withholds its hand-off, so that the bounded waits give up (failure test).
    p.relay_parts = 1;
    int want_relay = opts ? opts->relay : 0;
    if (want_relay < -8 || want_relay > 8 || want_relay == -1)
        return MAMBA_ERR_UNSUPPORTED;
    if (want_relay < 0) {
        p.relay_withhold = true;
        want_relay = -want_relay;
    }
    if (want_relay >= 2 && (p.family != Family::Scalar || spans != 1))
        return MAMBA_ERR_UNSUPPORTED;
    if (p.family == Family::Scalar && spans == 1 && seqlen > 0 && want_relay != 1) {
        const int64_t units = batch * ((d_inner + 63) / 64);
        int64_t rem = units % cus;
        int64_t k = 1, plen = 0;
        if (want_relay >= 2) {
            k = want_relay;
            if (rem == 0)
                rem = units;
            plen = (seqlen + k - 1) / k;
        } else if (units > cus && rem > 0 && rem * 2 <= cus && seqlen >= 512) {
            k = 2;
            plen = (seqlen + 1) / 2;
        }
        if (k >= 2) {
            plen = (plen + p.chunk - 1) / p.chunk * p.chunk;
            k = (seqlen + plen - 1) / plen; // every part non-empty
            if (k >= 2) {
                p.relay_parts = (int)k;
                p.relay_tiles = rem;
                p.relay_len = plen;
            }
        }
    }
    *plan = p;
    return MAMBA_OK;
}

// Workspace layout: [staged B/C (scalar family), 256-byte aligned] [span summaries].
size_t staged_bytes_for(int64_t batch, int64_t seqlen, int64_t d_state, const Plan &p)
{
    if (p.family != Family::Scalar || seqlen <= 0)
        return 0;
    const size_t rows = (size_t)seqlen + (size_t)p.chunk;
    const size_t per_row = 2 * (size_t)d_state + (p.rot ? (size_t)d_state / 2 : 0); // B, C, theta
    const size_t bytes = (size_t)batch * rows * per_row * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

// Relay area: [hand-off flags, fault word; 256-byte aligned][hand-off states].
size_t relay_sync_bytes(const Plan &p)
{
    if (p.relay_parts < 2)
        return 0;
    const size_t words = (size_t)p.relay_tiles * (size_t)(p.relay_parts - 1) + 1;
    return (words * sizeof(uint32_t) + 255) / 256 * 256;
}

size_t relay_state_bytes(int64_t d_state, const Plan &p)
{
    if (p.relay_parts < 2)
        return 0;
    return (size_t)p.relay_tiles * (size_t)(p.relay_parts - 1) * 64 * (size_t)d_state *
           sizeof(float);
}

size_t workspace_bytes_for(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                           const Plan &p)
{
    size_t n = staged_bytes_for(batch, seqlen, d_state, p);
    n += relay_sync_bytes(p) + relay_state_bytes(d_state, p);
    if (p.n_spans > 1) // decay [c][S], hloc [c][S], h_in [S][c] (+ rotation: 2x2 [pair][S])
        n += (size_t)(p.rot ? 5 : 3) * (size_t)p.n_spans * (size_t)(batch * d_inner * d_state) *
             sizeof(float);
    return n;
}

// Backward launch plan: the compiled variant's segment length, and the sequence split.
// Units of (batch row, 64-channel tile) run two blocks per compute unit.  The split costs
// two summary passes over the whole sequence (about a third more work) whatever the span
// count, so it is used only when the units cannot even give every compute unit one block,
// or (zero-order hold) when they overflow one round of two blocks per compute unit; then
// the sequence is cut into enough spans (a power of two, at most 64, each at least 64
// steps) for about four full rounds of blocks.
struct BwdPlan {
    int seg_len;
    int n_spans;
    int64_t span_len;
    int fwd_waves, fwd_chunk; // forward span-summary pass (scalar family)
    bool zoh;                 // zero-order-hold discretisation
};

mamba_status_t bwd_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                        const mamba_scan_opts_t *opts, BwdPlan *plan)
{
    BwdPlan p{};
    int waves = 0;
    if (!bwd_variant(d_state, &waves, &p.seg_len))
        return MAMBA_ERR_UNSUPPORTED;
    if (opts && (opts->chunk_len || opts->waves || opts->kernel || opts->relay ||
                 (opts->discretization != MAMBA_DISC_EULER &&
                  opts->discretization != MAMBA_DISC_ZOH)))
        return MAMBA_ERR_UNSUPPORTED;
    p.zoh = opts && opts->discretization == MAMBA_DISC_ZOH;
    const bool fixed = opts && opts->n_spans;
    if (fixed && (opts->n_spans < 1 || opts->n_spans > 64))
        return MAMBA_ERR_UNSUPPORTED;
    const int S = p.seg_len;
    int n = 1;
    if (fixed) {
        n = opts->n_spans;
    } else if (seqlen >= 128) {
        const int64_t units = batch * ((d_inner + 63) / 64);
        const int64_t cus = cu_count();
        // The zero-order hold's variant holds two blocks per compute unit: past one round of
        // them, the split also evens out the partial last round (640 units at the large
        // prefill: 7.8 ms unsplit, 6.7 / 6.4 / 6.5 ms in 2 / 4 / 8 spans).
        if (units < cus || (p.zoh && units > cus * 2)) {
            const int64_t want = cus * 2 /*blocks each*/ * 4 /*rounds*/;
            while (units * n < want && n < 64 && seqlen / (2 * n) >= 64)
                n *= 2;
        }
    }
    int64_t len = seqlen > 0 ? (seqlen + n - 1) / n : S;
    len = (len + S - 1) / S * S;
    if (len < S)
        len = S;
    n = seqlen > 0 ? (int)((seqlen + len - 1) / len) : 1;
    p.fwd_waves = scalar_default_waves(d_state);
    p.fwd_chunk = scalar_default_chunk(d_state);
    if (n > 1 && (!scalar_variant_supported(d_state, p.fwd_waves, p.fwd_chunk) ||
                  len % p.fwd_chunk != 0 || !scalar_span_ok(len, d_inner))) {
        if (fixed)
            return MAMBA_ERR_UNSUPPORTED;
        n = 1;
        len = (seqlen + S - 1) / S * S;
    }
    p.n_spans = n;
    p.span_len = len;
    *plan = p;
    return MAMBA_OK;
}

// Backward workspace: [segment checkpoints][dB/dC tile partials][dA partials]
// [dD, dbias partials] and, with spans, [staged B/C][forward span decay][forward span
// local state][state entering each span][adjoint decay][adjoint local][adjoint entering
// each span]; each region 256-byte aligned.  Offsets in bytes; off[11] is the total.
// With checkpoints from the forward pass (ext_ck) the checkpoint region and the forward
// span regions are empty.
void bwd_layout(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                const BwdPlan &p, bool ext_ck, size_t off[12])
{
    auto al = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t S = (size_t)p.seg_len;
    const size_t n_seg = (size_t)((seqlen + p.seg_len - 1) / p.seg_len);
    const size_t units = (size_t)batch * (size_t)((d_inner + 63) / 64);
    const size_t N = (size_t)d_state, f = sizeof(float);
    const size_t sp = (size_t)p.n_spans;
    const size_t bdn = (size_t)batch * (size_t)d_inner * N;
    size_t sz[11] = {};
    sz[0] = al(units * n_seg * N * 64 * f);
    sz[1] = al(units * (size_t)seqlen * 2 * N * f);
    sz[2] = al(sp * bdn * f);
    sz[3] = al(sp * (size_t)batch * (size_t)d_inner * 2 * f);
    if (p.n_spans > 1) {
        sz[4] = al((size_t)batch * ((size_t)seqlen + (size_t)p.fwd_chunk) * 2 * N * f);
        for (int i = 5; i < 11; ++i)
            sz[i] = al(sp * bdn * f);
    }
    if (ext_ck)
        sz[0] = sz[4] = sz[5] = sz[6] = sz[7] = 0;
    (void)S;
    off[0] = 0;
    for (int i = 0; i < 11; ++i)
        off[i + 1] = off[i] + sz[i];
    if (seqlen == 0)
        off[11] = 0;
}

mamba_status_t hip_status(hipError_t e) { return e == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP; }

} // namespace

extern "C" {

const char *mamba_status_string(mamba_status_t s)
{
    switch (s) {
    case MAMBA_OK: return "MAMBA_OK";
    case MAMBA_ERR_NULL_ARG: return "MAMBA_ERR_NULL_ARG: a required pointer is NULL";
    case MAMBA_ERR_BAD_SHAPE: return "MAMBA_ERR_BAD_SHAPE: negative or overflowing size";
    case MAMBA_ERR_BAD_DTYPE: return "MAMBA_ERR_BAD_DTYPE: unknown dtype";
    case MAMBA_ERR_UNSUPPORTED: return "MAMBA_ERR_UNSUPPORTED: d_state or option not supported";
    case MAMBA_ERR_MISALIGNED: return "MAMBA_ERR_MISALIGNED: pointer not aligned";
    case MAMBA_ERR_ALIASING: return "MAMBA_ERR_ALIASING: an output overlaps another argument";
    case MAMBA_ERR_WORKSPACE: return "MAMBA_ERR_WORKSPACE: workspace missing or too small";
    case MAMBA_ERR_HIP: return "MAMBA_ERR_HIP: HIP launch or runtime error";
    }
    return "MAMBA_ERR_UNKNOWN";
}

int32_t mamba_d_state_supported(int64_t d_state) { return padded_d_state(d_state) ? 1 : 0; }

size_t mamba_scan_fwd_workspace_size_ext(int64_t batch, int64_t seqlen, int64_t d_inner,
                                         int64_t d_state, const mamba_scan_ext_t *ext,
                                         const mamba_scan_opts_t *opts)
{
    int64_t tmp;
    const int64_t np = padded_d_state(d_state);
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 ||
        !mul_ok(batch, d_inner, &tmp) || !mul_ok(tmp, d_state, &tmp) || !np)
        return (size_t)-1;
    Rows rows;
    if (!rows_of(ext, d_inner, d_state, &rows))
        return (size_t)-1;
    Plan p;
    if (make_plan(batch, seqlen, d_inner, np, opts, ext, &p, &rows) != MAMBA_OK)
        return (size_t)-1;
    size_t pad = 0;
    if (np != d_state && seqlen > 0) {
        FwdPad f;
        // (the dtype is not known here: room for 4-byte elements)
        if (!fwd_pad_layout(batch, seqlen, d_inner, np, 4, ext && ext->theta,
                            ext && ext->lambda && ext->B_prev, &f))
            return (size_t)-1;
        pad = f.total;
    }
    return pad + workspace_bytes_for(batch, seqlen, d_inner, np, p);
}

size_t mamba_scan_fwd_workspace_size_ex(int64_t batch, int64_t seqlen, int64_t d_inner,
                                        int64_t d_state, const mamba_scan_opts_t *opts)
{
    return mamba_scan_fwd_workspace_size_ext(batch, seqlen, d_inner, d_state, nullptr, opts);
}

size_t mamba_scan_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner,
                                     int64_t d_state)
{
    return mamba_scan_fwd_workspace_size_ex(batch, seqlen, d_inner, d_state, nullptr);
}

mamba_status_t mamba_scan_fwd_ex(const void *u, const void *delta, const float *A,
                                 const void *B, const void *C, const float *D, const void *z,
                                 const float *delta_bias, const float *h0, void *y,
                                 float *h_last, int64_t batch, int64_t seqlen, int64_t d_inner,
                                 int64_t d_state, mamba_dtype_t dtype, void *workspace,
                                 size_t workspace_bytes, const mamba_scan_opts_t *opts,
                                 void *stream)
{
    return mamba_scan_fwd_ext(u, delta, A, B, C, D, z, delta_bias, h0, y, h_last, batch, seqlen,
                              d_inner, d_state, dtype, workspace, workspace_bytes, opts, nullptr,
                              stream);
}

} // extern "C"

// The forward scan: argument checks, then the launches.  check_only: run every check that
// does not involve the workspace and return before touching the device (the allocation-
// free entry point validates this way before it looks up its device array).
static mamba_status_t scan_fwd_impl(const void *u, const void *delta, const float *A,
                                    const void *B, const void *C, const float *D, const void *z,
                                    const float *delta_bias, const float *h0, void *y,
                                    float *h_last, int64_t batch, int64_t seqlen,
                                    int64_t d_inner, int64_t d_state, mamba_dtype_t dtype,
                                    void *workspace, size_t workspace_bytes,
                                    const mamba_scan_opts_t *opts, const mamba_scan_ext_t *ext,
                                    void *stream, bool check_only)
{
    const void *lam = ext ? ext->lambda : nullptr;
    const void *u_prev = lam ? ext->u_prev : nullptr; // used by the trapezoid only
    const void *B_prev = lam ? ext->B_prev : nullptr;
    const void *theta = ext ? ext->theta : nullptr;
    float *ckpt = ext ? ext->ckpt : nullptr;
    // ---- sizes and dtype ----
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16)
        return MAMBA_ERR_BAD_DTYPE;
    const int64_t np = padded_d_state(d_state); // the compiled size the scan runs at
    if (!np || (theta && d_state % 2 != 0))
        return MAMBA_ERR_UNSUPPORTED;
    const bool padded = np != d_state;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    int64_t bld, bln, bdn, dn, t;
    if (!mul_ok(batch, seqlen, &t) || !mul_ok(t, d_inner, &bld) || !mul_ok(bld, es, &t) ||
        !mul_ok(batch, seqlen, &t) || !mul_ok(t, d_state, &bln) || !mul_ok(bln, es, &t) ||
        !mul_ok(batch, d_inner, &t) || !mul_ok(t, d_state, &bdn) || !mul_ok(bdn, 4, &t) ||
        !mul_ok(d_inner, d_state, &dn) || !mul_ok(dn, 4, &t) || d_inner > INT32_MAX ||
        batch > INT32_MAX)
        return MAMBA_ERR_BAD_SHAPE;
    Rows rows;
    if (!rows_of(ext, d_inner, d_state, &rows))
        return MAMBA_ERR_BAD_SHAPE;
    // bytes spanned by each activation (its strided extent)
    const int64_t x_u = extent_bytes(batch * seqlen, rows.u, d_inner, es),
                  x_d = extent_bytes(batch * seqlen, rows.d, d_inner, es),
                  x_z = extent_bytes(batch * seqlen, rows.z, d_inner, es),
                  x_B = extent_bytes(batch * seqlen, rows.B, d_state, es),
                  x_C = extent_bytes(batch * seqlen, rows.C, d_state, es);
    if (x_u < 0 || x_d < 0 || x_z < 0 || x_B < 0 || x_C < 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (batch == 0 || d_inner == 0)
        return MAMBA_OK;

    // ---- required pointers ----
    const bool has_seq = seqlen > 0;
    if (!A || (has_seq && (!u || !delta || !B || !C || !y)))
        return MAMBA_ERR_NULL_ARG;

    // ---- alignment ----
    const void *elem_ptrs[] = {u, delta, B, C, z, y, lam, u_prev, B_prev, theta};
    for (const void *p : elem_ptrs)
        if (p && !aligned(p, (size_t)es))
            return MAMBA_ERR_MISALIGNED;
    const void *f32_ptrs[] = {A, D, delta_bias, h0, h_last, ckpt};
    for (const void *p : f32_ptrs)
        if (p && !aligned(p, 4))
            return MAMBA_ERR_MISALIGNED;

    // ---- plan and workspace ----
    Plan plan;
    const mamba_status_t ps = make_plan(batch, seqlen, d_inner, np, opts, ext, &plan, &rows);
    if (ps != MAMBA_OK)
        return ps;
    FwdPad pad{};
    if (padded && seqlen > 0 &&
        !fwd_pad_layout(batch, seqlen, d_inner, np, 4, theta != nullptr, B_prev != nullptr, &pad))
        return MAMBA_ERR_BAD_SHAPE;
    const size_t need = pad.total + workspace_bytes_for(batch, seqlen, d_inner, np, plan);
    if (!check_only && need > 0 && (!workspace || workspace_bytes < need))
        return MAMBA_ERR_WORKSPACE;
    if (!check_only && need > 0 && !aligned(workspace, 4))
        return MAMBA_ERR_MISALIGNED;

    // ---- aliasing ----
    const Range r_in[] = {range_of(u, x_u),            range_of(delta, x_d),
                          range_of(z, x_z),            range_of(B, x_B),
                          range_of(C, x_C),            range_of(A, dn * 4),
                          range_of(D, d_inner * 4),    range_of(delta_bias, d_inner * 4),
                          range_of(lam, bld * es),     range_of(u_prev, batch * d_inner * es),
                          range_of(B_prev, batch * d_state * es),
                          range_of(theta, bln / 2 * es)};
    const Range r_h0 = range_of(h0, bdn * 4);
    const Range r_y = range_of(has_seq ? y : nullptr, bld * es);
    const Range r_hl = range_of(h_last, bdn * 4);
    const Range r_ws = range_of(need > 0 && !check_only ? workspace : nullptr, (int64_t)need);
    const int64_t ckb = ckpt ? ckpt_bytes(batch, seqlen, d_inner, np) : 0;
    if (ckb < 0)
        return MAMBA_ERR_BAD_SHAPE;
    const Range r_ck = range_of(has_seq ? ckpt : nullptr, ckb);
    for (const Range &r : r_in) {
        if (overlaps(r_y, r) || overlaps(r_hl, r) || overlaps(r_ws, r) || overlaps(r_ck, r))
            return MAMBA_ERR_ALIASING;
    }
    if (overlaps(r_y, r_h0) || overlaps(r_y, r_hl) || overlaps(r_y, r_ws) ||
        overlaps(r_ws, r_h0) || overlaps(r_ws, r_hl) || overlaps(r_ck, r_y) ||
        overlaps(r_ck, r_h0) || overlaps(r_ck, r_hl) || overlaps(r_ck, r_ws))
        return MAMBA_ERR_ALIASING;
    if (overlaps(r_hl, r_h0) && (const void *)h_last != (const void *)h0)
        return MAMBA_ERR_ALIASING;
    if (check_only)
        return MAMBA_OK;

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);

    // ---- empty sequence: the final state is the initial state ----
    if (!has_seq) {
        if (h_last)
            return hip_status(launch_copy_state(h_last, h0, bdn, st));
        return MAMBA_OK;
    }

    char *ws_bytes = static_cast<char *>(workspace);
    float *hl_run = h_last; // the final state as the kernels write it
    if (padded) {
        // the state arrays as rows of np entries at the front of the workspace
        char *w = ws_bytes;
        const int32_t n32 = (int32_t)d_state, np32 = (int32_t)np, es32 = (int32_t)es;
        if (launch_pad_rows(w + pad.a, A, d_inner, n32, np32, 4, -1.0f, st) != hipSuccess ||
            launch_pad_rows(w + pad.b, B, batch * seqlen, n32, np32, es32, 0.0f, st,
                            rows.B) != hipSuccess ||
            launch_pad_rows(w + pad.c, C, batch * seqlen, n32, np32, es32, 0.0f, st,
                            rows.C) != hipSuccess)
            return MAMBA_ERR_HIP;
        rows.B = rows.C = np; // the copies are contiguous
        A = reinterpret_cast<const float *>(w + pad.a);
        B = w + pad.b;
        C = w + pad.c;
        if (h0) {
            if (launch_pad_rows(w + pad.h0, h0, batch * d_inner, n32, np32, 4, 0.0f, st) !=
                hipSuccess)
                return MAMBA_ERR_HIP;
            h0 = reinterpret_cast<const float *>(w + pad.h0);
        }
        if (h_last)
            hl_run = reinterpret_cast<float *>(w + pad.hl);
        if (theta) {
            if (launch_pad_rows(w + pad.theta, theta, batch * seqlen, n32 / 2, np32 / 2, es32,
                                0.0f, st) != hipSuccess)
                return MAMBA_ERR_HIP;
            theta = w + pad.theta;
        }
        if (B_prev) {
            if (launch_pad_rows(w + pad.bprev, B_prev, batch, n32, np32, es32, 0.0f, st) !=
                hipSuccess)
                return MAMBA_ERR_HIP;
            B_prev = w + pad.bprev;
        }
        ws_bytes += pad.total;
    }
    const int64_t N = np;              // the state size of every launch below
    const int64_t bdk = batch * d_inner * N;

    auto run = [&]() -> mamba_status_t {
    ScanLaunch L{};
    L.u = u;
    L.delta = delta;
    L.z = z;
    L.B = B;
    L.C = C;
    L.A = A;
    L.D = D;
    L.bias = delta_bias;
    L.y = y;
    L.h_last = hl_run;
    L.batch = batch;
    L.L = seqlen;
    L.d_inner = d_inner;
    L.d_state = N;
    L.span_len = plan.span_len;
    L.n_spans = plan.n_spans;
    L.waves = plan.waves;
    L.chunk = plan.chunk;
    L.dtype = dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32;
    L.zoh = plan.zoh;
    L.trap = plan.trap;
    L.rot = plan.rot;
    L.lam = lam;
    L.u_prev = u_prev;
    L.B_prev = B_prev;
    L.theta = theta;
    L.ckpt = plan.ckpt ? ckpt : nullptr;
    L.su = rows.u;
    L.sd = rows.d;
    L.sz = rows.z;
    L.sB = rows.B;
    L.sC = rows.C;

    auto full = [&](const ScanLaunch &x) {
        switch (plan.family) {
        case Family::Rows: return launch_rows_full(x, st);
        case Family::Scalar: return launch_scalar_full(x, st);
        default: return launch_scan_full(x, st);
        }
    };
    auto end = [&](const ScanLaunch &x) {
        switch (plan.family) {
        case Family::Rows: return launch_rows_end(x, st);
        case Family::Scalar: return launch_scalar_end(x, st);
        default: return launch_scan_end(x, st);
        }
    };

    const size_t staged = staged_bytes_for(batch, seqlen, N, plan);
    L.relay_parts = 1;
    if (plan.relay_parts > 1) {
        L.relay_sync = reinterpret_cast<uint32_t *>(ws_bytes + staged);
        L.relay_state = reinterpret_cast<float *>(ws_bytes + staged + relay_sync_bytes(plan));
        L.relay_tiles = (int32_t)plan.relay_tiles;
        L.relay_parts = plan.relay_parts;
        L.relay_len = plan.relay_len;
        L.relay_withhold = plan.relay_withhold;
        L.relay_max_polls = plan.relay_withhold ? kRelayTestPolls : kRelayPolls;
    }
    if (plan.family == Family::Scalar) {
        L.bc_staged = reinterpret_cast<float *>(ws_bytes);
        L.staged_rows = seqlen + plan.chunk;
        if (launch_stage_bc(L, st) != hipSuccess) // also clears the relay flags
            return MAMBA_ERR_HIP;
    }

    if (plan.n_spans == 1) {
        L.h_init = h0;
        L.h_init_span_stride = 0;
        L.first_span = 0;
        L.launch_spans = 1;
        return hip_status(full(L));
    }

    // ---- split sequence: span summaries, carry pass, full rescan ----
    const int64_t S = plan.n_spans;
    float *ws = reinterpret_cast<float *>(ws_bytes + staged); // (no relay with spans)
    float *ws_decay = ws;
    float *ws_hloc = ws + S * bdk;
    float *ws_hin = ws + 2 * S * bdk;
    float *ws_rot = plan.rot ? ws + 3 * S * bdk : nullptr; // (pairs * S * 4 = 2 * S * bdk)

    ScanLaunch E = L;
    E.h_init = nullptr;
    E.h_init_span_stride = 0;
    E.ckpt = nullptr; // span summaries hold local states: no checkpoints
    E.ws_decay = ws_decay;
    E.ws_hloc = ws_hloc;
    E.ws_rot = ws_rot;
    E.first_span = 0;
    E.launch_spans = (int32_t)(S - 1);
    hipError_t e = end(E);
    if (e != hipSuccess)
        return MAMBA_ERR_HIP;

    CarryLaunch K{};
    K.ws_decay = ws_decay;
    K.ws_hloc = ws_hloc;
    K.ws_rot = ws_rot;
    K.h0 = h0;
    K.h_in = ws_hin;
    K.columns = bdk;
    K.n_spans = (int32_t)S;
    e = launch_carry(K, st);
    if (e != hipSuccess)
        return MAMBA_ERR_HIP;

    L.h_init = ws_hin;
    L.h_init_span_stride = bdk;
    L.first_span = 0;
    L.launch_spans = (int32_t)S;
    return hip_status(full(L));
    };
    const mamba_status_t rs = run();
    if (rs != MAMBA_OK || !padded || !h_last)
        return rs;
    return hip_status(launch_unpad_rows(h_last, hl_run, batch * d_inner, (int32_t)d_state,
                                        (int32_t)N, 4, st));
}

// Checks of mamba_scan_fwd short of the workspace (for mamba_scan_fwd_noalloc).
mamba_status_t mamba_scan_fwd_check(const void *u, const void *delta, const float *A,
                                    const void *B, const void *C, const float *D, const void *z,
                                    const float *delta_bias, const float *h0, void *y,
                                    float *h_last, int64_t batch, int64_t seqlen,
                                    int64_t d_inner, int64_t d_state, mamba_dtype_t dtype)
{
    return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, h0, y, h_last, batch, seqlen,
                         d_inner, d_state, dtype, nullptr, 0, nullptr, nullptr, nullptr, true);
}

extern "C" {

mamba_status_t mamba_scan_fwd_ext(const void *u, const void *delta, const float *A,
                                  const void *B, const void *C, const float *D, const void *z,
                                  const float *delta_bias, const float *h0, void *y,
                                  float *h_last, int64_t batch, int64_t seqlen, int64_t d_inner,
                                  int64_t d_state, mamba_dtype_t dtype, void *workspace,
                                  size_t workspace_bytes, const mamba_scan_opts_t *opts,
                                  const mamba_scan_ext_t *ext, void *stream)
{
    return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, h0, y, h_last, batch, seqlen,
                         d_inner, d_state, dtype, workspace, workspace_bytes, opts, ext, stream,
                         false);
}

// Reads one fault word of a workspace back to the host (synchronises the stream).
static mamba_status_t read_fault_word(const uint32_t *word, uint32_t *out, void *stream)
{
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    uint32_t v = 0;
    if (hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return MAMBA_ERR_HIP;
    *out = v;
    return MAMBA_OK;
}

mamba_status_t mamba_scan_fwd_relay_faults(const void *workspace, size_t workspace_bytes,
                                           int64_t batch, int64_t seqlen, int64_t d_inner,
                                           int64_t d_state, const mamba_scan_opts_t *opts,
                                           const mamba_scan_ext_t *ext, uint32_t *faults,
                                           void *stream)
{
    if (!faults)
        return MAMBA_ERR_NULL_ARG;
    *faults = 0;
    int64_t t;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 || !mul_ok(batch, d_inner, &t) ||
        !mul_ok(t, d_state, &t))
        return MAMBA_ERR_BAD_SHAPE;
    const int64_t np = padded_d_state(d_state);
    if (!np)
        return MAMBA_ERR_UNSUPPORTED;
    Rows rows;
    if (!rows_of(ext, d_inner, d_state, &rows))
        return MAMBA_ERR_BAD_SHAPE;
    Plan plan;
    const mamba_status_t ps = make_plan(batch, seqlen, d_inner, np, opts, ext, &plan, &rows);
    if (ps != MAMBA_OK)
        return ps;
    if (plan.relay_parts < 2 || seqlen == 0 || batch == 0 || d_inner == 0)
        return MAMBA_OK; // no relay: nothing can have timed out
    FwdPad pad{};
    if (np != d_state &&
        !fwd_pad_layout(batch, seqlen, d_inner, np, 4, ext && ext->theta,
                        ext && ext->lambda && ext->B_prev, &pad))
        return MAMBA_ERR_BAD_SHAPE;
    const size_t need = pad.total + workspace_bytes_for(batch, seqlen, d_inner, np, plan);
    if (!workspace || workspace_bytes < need)
        return MAMBA_ERR_WORKSPACE;
    const size_t staged = pad.total + staged_bytes_for(batch, seqlen, np, plan);
    const uint32_t *word = reinterpret_cast<const uint32_t *>(
                               static_cast<const char *>(workspace) + staged) +
                           plan.relay_tiles * (plan.relay_parts - 1);
    return read_fault_word(word, faults, stream);
}

mamba_status_t mamba_scan_fwd(const void *u, const void *delta, const float *A, const void *B,
                              const void *C, const float *D, const void *z,
                              const float *delta_bias, const float *h0, void *y, float *h_last,
                              int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                              mamba_dtype_t dtype, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    return mamba_scan_fwd_ex(u, delta, A, B, C, D, z, delta_bias, h0, y, h_last, batch, seqlen,
                             d_inner, d_state, dtype, workspace, workspace_bytes, nullptr,
                             stream);
}

mamba_status_t mamba_state_update(float *h, const void *u, const void *delta, const float *A,
                                  const void *B, const void *C, const float *D, const void *z,
                                  const float *delta_bias, void *y, int64_t batch,
                                  int64_t d_inner, int64_t d_state, mamba_dtype_t dtype,
                                  void *stream)
{
    return mamba_state_update_ex(h, u, delta, A, B, C, D, z, delta_bias, y, batch, d_inner,
                                 d_state, dtype, MAMBA_DISC_EULER, stream);
}

mamba_status_t mamba_state_update_ex(float *h, const void *u, const void *delta,
                                     const float *A, const void *B, const void *C,
                                     const float *D, const void *z, const float *delta_bias,
                                     void *y, int64_t batch, int64_t d_inner, int64_t d_state,
                                     mamba_dtype_t dtype, int32_t discretization, void *stream)
{
    return mamba_state_update_ext(h, u, delta, A, B, C, D, z, delta_bias, y, batch, d_inner,
                                  d_state, dtype, discretization, nullptr, stream);
}

mamba_status_t mamba_state_update_ext(float *h, const void *u, const void *delta,
                                      const float *A, const void *B, const void *C,
                                      const float *D, const void *z, const float *delta_bias,
                                      void *y, int64_t batch, int64_t d_inner, int64_t d_state,
                                      mamba_dtype_t dtype, int32_t discretization,
                                      const mamba_scan_ext_t *ext, void *stream)
{
    const void *lam = ext ? ext->lambda : nullptr;
    const void *u_prev = lam ? ext->u_prev : nullptr;
    const void *B_prev = lam ? ext->B_prev : nullptr;
    const void *theta = ext ? ext->theta : nullptr;
    if (discretization != MAMBA_DISC_EULER && discretization != MAMBA_DISC_ZOH)
        return MAMBA_ERR_UNSUPPORTED;
    if ((lam && discretization == MAMBA_DISC_ZOH) || (theta && d_state % 2 != 0) ||
        (ext && ext->ckpt))
        return MAMBA_ERR_UNSUPPORTED; // (checkpoints belong to the scan)
    if (batch < 0 || d_inner < 0 || d_state <= 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16)
        return MAMBA_ERR_BAD_DTYPE;
    if (!padded_d_state(d_state))
        return MAMBA_ERR_UNSUPPORTED;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    // compiled sizes move the state in 16-byte vectors; the others in 4-byte elements
    const size_t h_align = d_state_ok(d_state) ? 16 : 4;
    int64_t bd, bn, bdn, dn, t;
    if (!mul_ok(batch, d_inner, &bd) || !mul_ok(bd, es, &t) || !mul_ok(batch, d_state, &bn) ||
        !mul_ok(bd, d_state, &bdn) || !mul_ok(bdn, 4, &t) || !mul_ok(d_inner, d_state, &dn) ||
        !mul_ok(dn, 4, &t) || d_inner > INT32_MAX / 64)
        return MAMBA_ERR_BAD_SHAPE;
    Rows rows; // strides between batch rows
    if (!rows_of(ext, d_inner, d_state, &rows))
        return MAMBA_ERR_BAD_SHAPE;
    const int64_t x_u = extent_bytes(batch, rows.u, d_inner, es),
                  x_d = extent_bytes(batch, rows.d, d_inner, es),
                  x_z = extent_bytes(batch, rows.z, d_inner, es),
                  x_B = extent_bytes(batch, rows.B, d_state, es),
                  x_C = extent_bytes(batch, rows.C, d_state, es);
    if (x_u < 0 || x_d < 0 || x_z < 0 || x_B < 0 || x_C < 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (batch == 0 || d_inner == 0)
        return MAMBA_OK;
    if (!h || !u || !delta || !A || !B || !C || !y)
        return MAMBA_ERR_NULL_ARG;

    const void *elem_ptrs[] = {u, delta, B, C, z, y, lam, u_prev, B_prev, theta};
    for (const void *p : elem_ptrs)
        if (p && !aligned(p, (size_t)es))
            return MAMBA_ERR_MISALIGNED;
    if (!aligned(h, h_align) || !aligned(A, h_align) || (D && !aligned(D, 4)) ||
        (delta_bias && !aligned(delta_bias, 4)))
        return MAMBA_ERR_MISALIGNED;

    const Range r_in[] = {range_of(u, x_u),           range_of(delta, x_d),
                          range_of(z, x_z),           range_of(B, x_B),
                          range_of(C, x_C),           range_of(A, dn * 4),
                          range_of(D, d_inner * 4),   range_of(delta_bias, d_inner * 4),
                          range_of(lam, bd * es),     range_of(u_prev, bd * es),
                          range_of(B_prev, bn * es),  range_of(theta, bn / 2 * es)};
    const Range r_h = range_of(h, bdn * 4);
    const Range r_y = range_of(y, bd * es);
    if (overlaps(r_h, r_y))
        return MAMBA_ERR_ALIASING;
    for (const Range &r : r_in)
        if (overlaps(r_h, r) || overlaps(r_y, r))
            return MAMBA_ERR_ALIASING;

    StepLaunch S{};
    S.h = h;
    S.u = u;
    S.delta = delta;
    S.z = z;
    S.B = B;
    S.C = C;
    S.A = A;
    S.D = D;
    S.bias = delta_bias;
    S.y = y;
    S.batch = batch;
    S.d_inner = d_inner;
    S.d_state = d_state;
    S.dtype = dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32;
    S.zoh = discretization == MAMBA_DISC_ZOH;
    S.trap = lam != nullptr;
    S.rot = theta != nullptr;
    S.lam = lam;
    S.u_prev = u_prev;
    S.B_prev = B_prev;
    S.theta = theta;
    S.su = rows.u;
    S.sd = rows.d;
    S.sz = rows.z;
    S.sB = rows.B;
    S.sC = rows.C;
    return hip_status(launch_state_update(S, reinterpret_cast<hipStream_t>(stream)));
}

mamba_status_t mamba_conv1d_silu_fwd(const void *x, const float *w, const float *conv_bias,
                                     const void *state_in, void *u, void *state_out,
                                     int64_t batch, int64_t seqlen, int64_t d_inner,
                                     int64_t d_conv, mamba_dtype_t dtype, void *stream)
{
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_conv < 1)
        return MAMBA_ERR_BAD_SHAPE;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16)
        return MAMBA_ERR_BAD_DTYPE;
    if (d_conv < 2 || d_conv > 4)
        return MAMBA_ERR_UNSUPPORTED;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    int64_t bld, bds, dk, t;
    if (!mul_ok(batch, seqlen, &t) || !mul_ok(t, d_inner, &bld) || !mul_ok(bld, es, &t) ||
        !mul_ok(batch, d_inner, &t) || !mul_ok(t, d_conv - 1, &bds) || !mul_ok(bds, es, &t) ||
        !mul_ok(d_inner, d_conv, &dk) || !mul_ok(dk, 4, &t) || d_inner > INT32_MAX ||
        batch > 65535 || (seqlen + 127) / 128 > 65535)
        return MAMBA_ERR_BAD_SHAPE;
    if (batch == 0 || d_inner == 0)
        return MAMBA_OK;
    if (!w || (seqlen > 0 && (!x || !u)))
        return MAMBA_ERR_NULL_ARG;
    if (!aligned(x, es) || !aligned(u, es) || !aligned(state_in, es) ||
        !aligned(state_out, es) || !aligned(w, 4) || (conv_bias && !aligned(conv_bias, 4)))
        return MAMBA_ERR_MISALIGNED;
    const Range r_x = range_of(x, bld * es), r_u = range_of(u, bld * es);
    const Range r_w = range_of(w, dk * 4), r_b = range_of(conv_bias, d_inner * 4);
    const Range r_si = range_of(state_in, bds * es), r_so = range_of(state_out, bds * es);
    if (overlaps(r_u, r_x) || overlaps(r_u, r_w) || overlaps(r_u, r_b) || overlaps(r_u, r_si) ||
        overlaps(r_u, r_so) || overlaps(r_so, r_x) || overlaps(r_so, r_w) || overlaps(r_so, r_b))
        return MAMBA_ERR_ALIASING;
    if (overlaps(r_si, r_so) && state_in != state_out)
        return MAMBA_ERR_ALIASING;

    ConvLaunch P{};
    P.x = x;
    P.w = w;
    P.bias = conv_bias;
    P.state_in = state_in;
    P.u = u;
    P.state_out = state_out;
    P.batch = batch;
    P.L = seqlen;
    P.d_inner = d_inner;
    P.d_conv = d_conv;
    P.dtype = dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32;
    P.vec4 = d_inner % 4 == 0 && aligned(x, 4 * es) && aligned(u, 4 * es);
    // (with seqlen == 0 the kernel only passes the state through)
    if (seqlen == 0 && (!state_out || state_out == state_in))
        return MAMBA_OK;
    return hip_status(launch_conv1d_silu(P, reinterpret_cast<hipStream_t>(stream)));
}

mamba_status_t mamba_conv1d_silu_update(void *state, const void *x, const float *w,
                                        const float *conv_bias, void *u, int64_t batch,
                                        int64_t d_inner, int64_t d_conv, mamba_dtype_t dtype,
                                        void *stream)
{
    if (batch < 0 || d_inner < 0 || d_conv < 1)
        return MAMBA_ERR_BAD_SHAPE;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16)
        return MAMBA_ERR_BAD_DTYPE;
    if (d_conv < 2 || d_conv > 4)
        return MAMBA_ERR_UNSUPPORTED;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    int64_t bd, bds, dk, t;
    if (!mul_ok(batch, d_inner, &bd) || !mul_ok(bd, es, &t) || !mul_ok(bd, d_conv - 1, &bds) ||
        !mul_ok(bds, es, &t) || !mul_ok(d_inner, d_conv, &dk) || !mul_ok(dk, 4, &t) ||
        d_inner > INT32_MAX)
        return MAMBA_ERR_BAD_SHAPE;
    if (bd == 0)
        return MAMBA_OK;
    if (!state || !x || !w || !u)
        return MAMBA_ERR_NULL_ARG;
    if (!aligned(state, es) || !aligned(x, es) || !aligned(u, es) || !aligned(w, 4) ||
        (conv_bias && !aligned(conv_bias, 4)))
        return MAMBA_ERR_MISALIGNED;
    const Range r_s = range_of(state, bds * es), r_x = range_of(x, bd * es);
    const Range r_u = range_of(u, bd * es), r_w = range_of(w, dk * 4);
    const Range r_b = range_of(conv_bias, d_inner * 4);
    if (overlaps(r_u, r_s) || overlaps(r_u, r_x) || overlaps(r_u, r_w) || overlaps(r_u, r_b) ||
        overlaps(r_s, r_x) || overlaps(r_s, r_w) || overlaps(r_s, r_b))
        return MAMBA_ERR_ALIASING;
    ConvLaunch P{};
    P.x = x;
    P.w = w;
    P.bias = conv_bias;
    P.u = u;
    P.state_out = state;
    P.batch = batch;
    P.d_inner = d_inner;
    P.d_conv = d_conv;
    P.dtype = dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32;
    return hip_status(launch_conv1d_silu_update(P, reinterpret_cast<hipStream_t>(stream)));
}


static size_t bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner,
                                 int64_t d_state, const mamba_scan_opts_t *opts, bool ext_ck)
{
    int64_t t;
    const int64_t np = padded_d_state(d_state);
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 || !np ||
        !mul_ok(batch, seqlen, &t) || !mul_ok(t, d_inner, &t) || !mul_ok(t, np, &t) ||
        !mul_ok(t, 8, &t))
        return (size_t)-1;
    BwdPlan plan;
    if (bwd_plan(batch, seqlen, d_inner, np, opts, &plan) != MAMBA_OK)
        return (size_t)-1;
    size_t off[12];
    bwd_layout(batch, seqlen, d_inner, np, plan, ext_ck, off);
    BwdPad pad{};
    if (np != d_state && seqlen > 0 && !bwd_pad_layout(batch, seqlen, d_inner, np, &pad))
        return (size_t)-1;
    return pad.total + off[11];
}

size_t mamba_scan_bwd_workspace_size_ex(int64_t batch, int64_t seqlen, int64_t d_inner,
                                        int64_t d_state, const mamba_scan_opts_t *opts)
{
    return bwd_workspace_size(batch, seqlen, d_inner, d_state, opts, false);
}

size_t mamba_scan_bwd_ckpt_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner,
                                          int64_t d_state, const mamba_scan_opts_t *opts)
{
    return bwd_workspace_size(batch, seqlen, d_inner, d_state, opts, true);
}

size_t mamba_scan_ckpt_size(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state)
{
    const int64_t np = padded_d_state(d_state);
    if (batch < 0 || seqlen < 0 || d_inner < 0 || !bwd_d_state_ok(np))
        return (size_t)-1;
    const int64_t b = ckpt_bytes(batch, seqlen, d_inner, np);
    return b < 0 ? (size_t)-1 : (size_t)b;
}

size_t mamba_scan_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner,
                                     int64_t d_state)
{
    return mamba_scan_bwd_workspace_size_ex(batch, seqlen, d_inner, d_state, nullptr);
}

mamba_status_t mamba_scan_bwd(const void *u, const void *delta, const float *A, const void *B,
                              const void *C, const float *D, const void *z,
                              const float *delta_bias, const float *h0, const void *dy,
                              const float *dh_last, void *du, void *ddelta, float *dA,
                              void *dB, void *dC, float *dD, void *dz, float *d_delta_bias,
                              float *dh0, int64_t batch, int64_t seqlen, int64_t d_inner,
                              int64_t d_state, mamba_dtype_t dtype, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    return mamba_scan_bwd_ex(u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_last, du, ddelta,
                             dA, dB, dC, dD, dz, d_delta_bias, dh0, batch, seqlen, d_inner,
                             d_state, dtype, workspace, workspace_bytes, nullptr, stream);
}

// The backward pass; ckpt: checkpoints written by the forward pass, or NULL (then the
// backward runs its own forward pass into the workspace).
static mamba_status_t bwd_impl(const void *u, const void *delta, const float *A, const void *B,
                               const void *C, const float *D, const void *z,
                               const float *delta_bias, const float *h0, const void *dy,
                               const float *dh_last, const float *ckpt, void *du, void *ddelta,
                               float *dA, void *dB, void *dC, float *dD, void *dz,
                               float *d_delta_bias, float *dh0, int64_t batch, int64_t seqlen,
                               int64_t d_inner, int64_t d_state, mamba_dtype_t dtype,
                               void *workspace, size_t workspace_bytes,
                               const mamba_scan_opts_t *opts, void *stream)
{
    // ---- sizes and dtype ----
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16)
        return MAMBA_ERR_BAD_DTYPE;
    const int64_t np = padded_d_state(d_state); // the compiled size the kernels run at
    if (!np)
        return MAMBA_ERR_UNSUPPORTED;
    const bool padded = np != d_state;
    BwdPlan plan;
    const mamba_status_t ps = bwd_plan(batch, seqlen, d_inner, np, opts, &plan);
    if (ps != MAMBA_OK)
        return ps;
    const int S = plan.seg_len;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    int64_t bld, bln, bdn, dn, t;
    if (!mul_ok(batch, seqlen, &t) || !mul_ok(t, d_inner, &bld) || !mul_ok(bld, es, &t) ||
        !mul_ok(batch, seqlen, &t) || !mul_ok(t, d_state, &bln) || !mul_ok(bln, es, &t) ||
        !mul_ok(bld, d_state, &t) || !mul_ok(t, 8, &t) || !mul_ok(batch, d_inner, &t) ||
        !mul_ok(t, d_state, &bdn) || !mul_ok(bdn, 4, &t) || !mul_ok(d_inner, d_state, &dn) ||
        !mul_ok(dn, 4, &t) || d_inner > INT32_MAX || batch > INT32_MAX ||
        (seqlen + S - 1) / S > INT32_MAX || plan.span_len > INT32_MAX)
        return MAMBA_ERR_BAD_SHAPE;
    if (batch == 0 || d_inner == 0)
        return MAMBA_OK;

    // ---- required pointers ----
    const bool has_seq = seqlen > 0;
    const bool ext_ck = ckpt != nullptr;
    if (!A || (has_seq && (!u || !delta || !B || !C || !dy || !du || !ddelta)) ||
        (has_seq && z && !dz))
        return MAMBA_ERR_NULL_ARG;
    if (!z)
        dz = nullptr; // no gate: there is no dz to write

    // ---- alignment ----
    const void *elem_ptrs[] = {u, delta, B, C, z, dy, du, ddelta, dB, dC, dz};
    for (const void *p : elem_ptrs)
        if (p && !aligned(p, (size_t)es))
            return MAMBA_ERR_MISALIGNED;
    const void *f32_ptrs[] = {A, D, delta_bias, h0, dh_last, dA, dD, d_delta_bias, dh0, ckpt};
    for (const void *p : f32_ptrs)
        if (p && !aligned(p, 4))
            return MAMBA_ERR_MISALIGNED;
    const int64_t ckb = ext_ck ? ckpt_bytes(batch, seqlen, d_inner, np) : 0;
    if (ckb < 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (ext_ck && (S != 8 || plan.zoh))
        return MAMBA_ERR_UNSUPPORTED; // the forward stores the state every 8 steps, for Euler

    // ---- workspace ----
    size_t off[12];
    bwd_layout(batch, seqlen, d_inner, np, plan, ext_ck, off);
    BwdPad pad{};
    if (padded && has_seq && !bwd_pad_layout(batch, seqlen, d_inner, np, &pad))
        return MAMBA_ERR_BAD_SHAPE;
    const size_t need = pad.total + off[11];
    if (need > 0 && (!workspace || workspace_bytes < need))
        return MAMBA_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 4))
        return MAMBA_ERR_MISALIGNED;

    // ---- aliasing: every output is disjoint from every input and every other output ----
    const Range r_in[] = {range_of(u, bld * es),       range_of(delta, bld * es),
                          range_of(z, bld * es),       range_of(dy, bld * es),
                          range_of(B, bln * es),       range_of(C, bln * es),
                          range_of(A, dn * 4),         range_of(D, d_inner * 4),
                          range_of(delta_bias, d_inner * 4), range_of(h0, bdn * 4),
                          range_of(dh_last, bdn * 4),
                          range_of(has_seq ? ckpt : nullptr, ckb)};
    const Range r_out[] = {range_of(has_seq ? du : nullptr, bld * es),
                           range_of(has_seq ? ddelta : nullptr, bld * es),
                           range_of(has_seq ? dz : nullptr, bld * es),
                           range_of(has_seq ? dB : nullptr, bln * es),
                           range_of(has_seq ? dC : nullptr, bln * es),
                           range_of(dA, dn * 4),
                           range_of(dD, d_inner * 4),
                           range_of(d_delta_bias, d_inner * 4),
                           range_of(dh0, bdn * 4),
                           range_of(need > 0 ? workspace : nullptr, (int64_t)need)};
    const int n_out = (int)(sizeof(r_out) / sizeof(r_out[0]));
    for (int i = 0; i < n_out; ++i) {
        for (const Range &r : r_in)
            if (overlaps(r_out[i], r))
                return MAMBA_ERR_ALIASING;
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(r_out[i], r_out[j]))
                return MAMBA_ERR_ALIASING;
    }

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);

    // ---- empty sequence: dh0 = dh_last, parameter gradients zero ----
    if (!has_seq) {
        hipError_t e = hipSuccess;
        if (dh0)
            e = launch_copy_state(dh0, dh_last, bdn, st);
        if (e == hipSuccess && dA)
            e = launch_copy_state(dA, nullptr, dn, st);
        if (e == hipSuccess && dD)
            e = launch_copy_state(dD, nullptr, d_inner, st);
        if (e == hipSuccess && d_delta_bias)
            e = launch_copy_state(d_delta_bias, nullptr, d_inner, st);
        return hip_status(e);
    }

    char *ws = static_cast<char *>(workspace);
    // a d_state without kernels of its own: the state-indexed inputs padded to np entries
    // per row at the front of the workspace, the state-indexed gradients written there
    // and copied back at the end
    void *dB_out = dB, *dC_out = dC;
    float *dA_out = dA, *dh0_out = dh0;
    const int64_t n_real = d_state;
    if (padded) {
        const int32_t n32 = (int32_t)d_state, np32 = (int32_t)np, es32 = (int32_t)es;
        if (launch_pad_rows(ws + pad.a, A, d_inner, n32, np32, 4, -1.0f, st) != hipSuccess ||
            launch_pad_rows(ws + pad.b, B, batch * seqlen, n32, np32, es32, 0.0f, st) != hipSuccess ||
            launch_pad_rows(ws + pad.c, C, batch * seqlen, n32, np32, es32, 0.0f, st) != hipSuccess)
            return MAMBA_ERR_HIP;
        A = reinterpret_cast<const float *>(ws + pad.a);
        B = ws + pad.b;
        C = ws + pad.c;
        if (h0) {
            if (launch_pad_rows(ws + pad.h0, h0, batch * d_inner, n32, np32, 4, 0.0f, st) !=
                hipSuccess)
                return MAMBA_ERR_HIP;
            h0 = reinterpret_cast<const float *>(ws + pad.h0);
        }
        if (dh_last) {
            if (launch_pad_rows(ws + pad.dhl, dh_last, batch * d_inner, n32, np32, 4, 0.0f, st) !=
                hipSuccess)
                return MAMBA_ERR_HIP;
            dh_last = reinterpret_cast<const float *>(ws + pad.dhl);
        }
        if (dB)
            dB = ws + pad.db;
        if (dC)
            dC = ws + pad.dc;
        if (dA)
            dA = reinterpret_cast<float *>(ws + pad.da);
        if (dh0)
            dh0 = reinterpret_cast<float *>(ws + pad.dh0);
        ws += pad.total;
        d_state = np;
        bdn = batch * d_inner * np;
    }
    const DType dt = dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32;
    auto region = [&](int i) { return reinterpret_cast<float *>(ws + off[i]); };

    BwdLaunch P{};
    if (plan.n_spans > 1 && ext_ck) {
        // the state entering each span is a checkpoint; only the adjoint carries are needed
        P.mu_dec = region(8);
        P.mu_loc = region(9);
        P.mu_in = region(10);
    } else if (plan.n_spans > 1) {
        // forward span summaries (the forward's span pass), then the state entering each span
        ScanLaunch E{};
        E.u = u;
        E.delta = delta;
        E.B = B;
        E.C = C;
        E.A = A;
        E.D = D;
        E.bias = delta_bias;
        E.ws_decay = region(5);
        E.ws_hloc = region(6);
        E.batch = batch;
        E.L = seqlen;
        E.d_inner = d_inner;
        E.d_state = d_state;
        E.span_len = plan.span_len;
        E.n_spans = plan.n_spans;
        E.first_span = 0;
        E.launch_spans = plan.n_spans - 1;
        E.waves = plan.fwd_waves;
        E.chunk = plan.fwd_chunk;
        E.dtype = dt;
        E.bc_staged = region(4);
        E.staged_rows = seqlen + plan.fwd_chunk;
        E.relay_parts = 1;
        E.su = E.sd = E.sz = d_inner;
        E.sB = E.sC = d_state;
        E.zoh = plan.zoh;
        if (launch_stage_bc(E, st) != hipSuccess || launch_scalar_end(E, st) != hipSuccess)
            return MAMBA_ERR_HIP;
        CarryLaunch K{};
        K.ws_decay = region(5);
        K.ws_hloc = region(6);
        K.h0 = h0;
        K.h_in = region(7);
        K.columns = bdn;
        K.n_spans = plan.n_spans;
        if (launch_carry(K, st) != hipSuccess)
            return MAMBA_ERR_HIP;
        P.h_in = region(7);
        P.mu_dec = region(8);
        P.mu_loc = region(9);
        P.mu_in = region(10);
    }
    P.n_spans = plan.n_spans;
    P.span_len = plan.span_len;
    P.u = u;
    P.delta = delta;
    P.z = z;
    P.dy = dy;
    P.B = B;
    P.C = C;
    P.A = A;
    P.D = D;
    P.bias = delta_bias;
    P.h0 = h0;
    P.dh_last = dh_last;
    P.du = du;
    P.ddelta = ddelta;
    P.dz = dz;
    P.dB = dB;
    P.dC = dC;
    P.dA = dA;
    P.dD = dD;
    P.dbias = d_delta_bias;
    P.dh0 = dh0;
    P.ckpt = ext_ck ? const_cast<float *>(ckpt) : region(0);
    P.ck_ext = ext_ck;
    P.dbc_part = region(1);
    P.dA_part = region(2);
    P.dDb_part = region(3);
    P.batch = batch;
    P.L = seqlen;
    P.d_inner = d_inner;
    P.d_state = d_state;
    P.dtype = dt;
    P.zoh = plan.zoh;
    if (launch_scan_bwd(P, st) != hipSuccess)
        return MAMBA_ERR_HIP;
    if (!padded)
        return MAMBA_OK;
    // the state-indexed gradients back to rows of the caller's d_state
    const int32_t nr = (int32_t)n_real, np32 = (int32_t)np, es32 = (int32_t)es;
    hipError_t e = hipSuccess;
    if (dB_out)
        e = launch_unpad_rows(dB_out, dB, batch * seqlen, nr, np32, es32, st);
    if (e == hipSuccess && dC_out)
        e = launch_unpad_rows(dC_out, dC, batch * seqlen, nr, np32, es32, st);
    if (e == hipSuccess && dA_out)
        e = launch_unpad_rows(dA_out, dA, d_inner, nr, np32, 4, st);
    if (e == hipSuccess && dh0_out)
        e = launch_unpad_rows(dh0_out, dh0, batch * d_inner, nr, np32, 4, st);
    return hip_status(e);
}

mamba_status_t mamba_scan_bwd_ex(const void *u, const void *delta, const float *A,
                                 const void *B, const void *C, const float *D, const void *z,
                                 const float *delta_bias, const float *h0, const void *dy,
                                 const float *dh_last, void *du, void *ddelta, float *dA,
                                 void *dB, void *dC, float *dD, void *dz, float *d_delta_bias,
                                 float *dh0, int64_t batch, int64_t seqlen, int64_t d_inner,
                                 int64_t d_state, mamba_dtype_t dtype, void *workspace,
                                 size_t workspace_bytes, const mamba_scan_opts_t *opts,
                                 void *stream)
{
    return bwd_impl(u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_last, nullptr, du, ddelta,
                    dA, dB, dC, dD, dz, d_delta_bias, dh0, batch, seqlen, d_inner, d_state,
                    dtype, workspace, workspace_bytes, opts, stream);
}

// ---- backward with the Mamba-3 options (scan_bwd_m3.hip) ----

// Options of a backward call with lambda or theta: Euler or (rotation only) the zero-order
// hold, at most 64 spans, d_state 4..32 compiled, contiguous inputs, no stored checkpoints.
static mamba_status_t m3_bwd_check(int64_t d_state, const mamba_scan_ext_t *ext,
                                   const mamba_scan_opts_t *opts, bool *zoh)
{
    *zoh = false;
    if (!bwd_d_state_ok(d_state) || (ext->theta && d_state % 2 != 0) || ext->ckpt ||
        ext->u_stride || ext->delta_stride || ext->z_stride || ext->B_stride || ext->C_stride)
        return MAMBA_ERR_UNSUPPORTED;
    if (opts) {
        if (opts->chunk_len || opts->waves || opts->kernel || opts->relay || opts->n_spans > 64 ||
            opts->n_spans < 0 ||
            (opts->discretization != MAMBA_DISC_EULER && opts->discretization != MAMBA_DISC_ZOH))
            return MAMBA_ERR_UNSUPPORTED;
        *zoh = opts->discretization == MAMBA_DISC_ZOH;
    }
    if (*zoh && ext->lambda)
        return MAMBA_ERR_UNSUPPORTED; // the trapezoid replaces the input term
    return MAMBA_OK;
}

// Sequence split of the Mamba-3 backward.  One block per (span, batch row, 64-channel tile);
// the kernel holds about three blocks per compute unit, so when the units alone leave compute
// units idle the sequence is cut into spans (powers of two, at least 64 steps each) for about
// two rounds of blocks.  A split needs the forward span pass of the scalar family with the same
// options (with the rotation: whole state pairs per wave, d_state 16 or 32); without it the
// call runs unsplit (automatic) or returns MAMBA_ERR_UNSUPPORTED (a requested split).
static mamba_status_t m3_plan(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                              bool rot, const mamba_scan_opts_t *opts, M3Plan *plan)
{
    M3Plan p{};
    p.fwd_waves = scalar_default_waves(d_state);
    p.fwd_chunk = scalar_default_chunk(d_state);
    const bool fixed = opts && opts->n_spans > 0;
    int n = fixed ? opts->n_spans : 1;
    if (!fixed && seqlen >= 128) {
        const int64_t units = batch * ((d_inner + 63) / 64);
        const int64_t cus = cu_count();
        if (units < cus) {
            const int64_t want = cus * 3 /*blocks each*/ * 2 /*rounds*/;
            while (units * n < want && n < 64 && seqlen / (2 * n) >= 64)
                n *= 2;
        }
    }
    constexpr int64_t kSeg = 8; // the kernel's segment between stored states
    int64_t len = seqlen > 0 ? (seqlen + n - 1) / n : kSeg;
    len = (len + kSeg - 1) / kSeg * kSeg;
    n = seqlen > 0 ? (int)((seqlen + len - 1) / len) : 1;
    if (n > 1 && (!scalar_variant_supported(d_state, p.fwd_waves, p.fwd_chunk) ||
                  (rot && (d_state / p.fwd_waves) % 2 != 0) || len % p.fwd_chunk != 0 ||
                  !scalar_span_ok(len, d_inner))) {
        if (fixed)
            return MAMBA_ERR_UNSUPPORTED;
        n = 1;
    }
    p.n_spans = n;
    p.span_len = n > 1 ? len : seqlen;
    *plan = p;
    return MAMBA_OK;
}

size_t mamba_scan_bwd_ext_workspace_size(int64_t batch, int64_t seqlen, int64_t d_inner,
                                         int64_t d_state, const mamba_scan_ext_t *ext,
                                         const mamba_scan_opts_t *opts)
{
    if (!ext || (!ext->lambda && !ext->theta))
        return bwd_workspace_size(batch, seqlen, d_inner, d_state, opts, false);
    int64_t t;
    bool zoh;
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0 || !mul_ok(batch, seqlen, &t) ||
        !mul_ok(t, d_inner, &t) || !mul_ok(t, d_state, &t) || !mul_ok(t, 8, &t) ||
        m3_bwd_check(d_state, ext, opts, &zoh) != MAMBA_OK)
        return (size_t)-1;
    M3Plan plan;
    if (m3_plan(batch, seqlen, d_inner, d_state, ext->theta != nullptr, opts, &plan) != MAMBA_OK)
        return (size_t)-1;
    size_t off[15];
    return m3_bwd_workspace_bytes(batch, seqlen, d_inner, d_state, ext->theta != nullptr, plan,
                                  off);
}

mamba_status_t mamba_scan_bwd_ext(const void *u, const void *delta, const float *A,
                                  const void *B, const void *C, const float *D, const void *z,
                                  const float *delta_bias, const float *h0, const void *dy,
                                  const float *dh_last, void *du, void *ddelta, float *dA,
                                  void *dB, void *dC, float *dD, void *dz, float *d_delta_bias,
                                  float *dh0, const mamba_scan_ext_t *ext,
                                  const mamba_scan_ext_grads_t *eg, int64_t batch,
                                  int64_t seqlen, int64_t d_inner, int64_t d_state,
                                  mamba_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                  const mamba_scan_opts_t *opts, void *stream)
{
    if (!ext || (!ext->lambda && !ext->theta)) {
        if (ext && (ext->ckpt || ext->u_stride || ext->delta_stride || ext->z_stride ||
                    ext->B_stride || ext->C_stride))
            return MAMBA_ERR_UNSUPPORTED;
        return bwd_impl(u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_last, nullptr, du,
                        ddelta, dA, dB, dC, dD, dz, d_delta_bias, dh0, batch, seqlen, d_inner,
                        d_state, dtype, workspace, workspace_bytes, opts, stream);
    }
    const void *lam = ext->lambda, *theta = ext->theta;
    const void *u_prev = lam ? ext->u_prev : nullptr, *B_prev = lam ? ext->B_prev : nullptr;
    void *dlam = eg ? eg->dlam : nullptr, *du_prev = eg ? eg->du_prev : nullptr;
    void *dB_prev = eg ? eg->dB_prev : nullptr, *dtheta = eg ? eg->dtheta : nullptr;
    if (!lam)
        dlam = du_prev = dB_prev = nullptr;
    if (!theta)
        dtheta = nullptr;
    // ---- sizes, dtype, options ----
    if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state <= 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16)
        return MAMBA_ERR_BAD_DTYPE;
    bool zoh;
    const mamba_status_t cs = m3_bwd_check(d_state, ext, opts, &zoh);
    if (cs != MAMBA_OK)
        return cs;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    int64_t bld, bln, bdn, dn, t;
    if (!mul_ok(batch, seqlen, &t) || !mul_ok(t, d_inner, &bld) || !mul_ok(bld, es, &t) ||
        !mul_ok(batch, seqlen, &t) || !mul_ok(t, d_state, &bln) || !mul_ok(bln, es, &t) ||
        !mul_ok(bld, d_state, &t) || !mul_ok(t, 8, &t) || !mul_ok(batch, d_inner, &t) ||
        !mul_ok(t, d_state, &bdn) || !mul_ok(bdn, 4, &t) || !mul_ok(d_inner, d_state, &dn) ||
        !mul_ok(dn, 4, &t) || d_inner > INT32_MAX || batch > INT32_MAX ||
        batch * ((d_inner + 63) / 64) > INT32_MAX)
        return MAMBA_ERR_BAD_SHAPE;
    if (batch == 0 || d_inner == 0)
        return MAMBA_OK;
    // ---- pointers ----
    const bool has_seq = seqlen > 0;
    if (!A || (has_seq && (!u || !delta || !B || !C || !dy || !du || !ddelta)) ||
        (has_seq && z && !dz))
        return MAMBA_ERR_NULL_ARG;
    if (!z)
        dz = nullptr;
    const void *elem_ptrs[] = {u, delta, B, C, z, dy, du, ddelta, dB, dC, dz, lam, u_prev,
                               B_prev, theta, dlam, du_prev, dB_prev, dtheta};
    for (const void *pp : elem_ptrs)
        if (pp && !aligned(pp, (size_t)es))
            return MAMBA_ERR_MISALIGNED;
    const void *f32_ptrs[] = {A, D, delta_bias, h0, dh_last, dA, dD, d_delta_bias, dh0};
    for (const void *pp : f32_ptrs)
        if (pp && !aligned(pp, 4))
            return MAMBA_ERR_MISALIGNED;
    const void *vec_ptrs[] = {B, C, B_prev, theta}; // a lane's states read as one vector
    for (const void *pp : vec_ptrs)
        if (pp && !aligned(pp, 16))
            return MAMBA_ERR_MISALIGNED;
    M3Plan plan;
    const mamba_status_t ps = m3_plan(batch, seqlen, d_inner, d_state, theta != nullptr, opts,
                                      &plan);
    if (ps != MAMBA_OK)
        return ps;
    size_t off[15];
    const size_t need = m3_bwd_workspace_bytes(batch, seqlen, d_inner, d_state, theta != nullptr,
                                               plan, off);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return MAMBA_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 4))
        return MAMBA_ERR_MISALIGNED;
    // ---- aliasing: every output is disjoint from every input and every other output ----
    const int64_t bd = batch * d_inner, bn = batch * d_state;
    const Range r_in[] = {range_of(u, bld * es),           range_of(delta, bld * es),
                          range_of(z, bld * es),           range_of(dy, bld * es),
                          range_of(B, bln * es),           range_of(C, bln * es),
                          range_of(A, dn * 4),             range_of(D, d_inner * 4),
                          range_of(delta_bias, d_inner * 4), range_of(h0, bdn * 4),
                          range_of(dh_last, bdn * 4),      range_of(lam, bld * es),
                          range_of(u_prev, bd * es),       range_of(B_prev, bn * es),
                          range_of(theta, bln / 2 * es)};
    const Range r_out[] = {range_of(has_seq ? du : nullptr, bld * es),
                           range_of(has_seq ? ddelta : nullptr, bld * es),
                           range_of(has_seq ? dz : nullptr, bld * es),
                           range_of(has_seq ? dB : nullptr, bln * es),
                           range_of(has_seq ? dC : nullptr, bln * es),
                           range_of(dA, dn * 4),
                           range_of(dD, d_inner * 4),
                           range_of(d_delta_bias, d_inner * 4),
                           range_of(dh0, bdn * 4),
                           range_of(has_seq ? dlam : nullptr, bld * es),
                           range_of(du_prev, bd * es),
                           range_of(dB_prev, bn * es),
                           range_of(has_seq ? dtheta : nullptr, bln / 2 * es),
                           range_of(need > 0 ? workspace : nullptr, (int64_t)need)};
    const int n_out = (int)(sizeof(r_out) / sizeof(r_out[0]));
    for (int i = 0; i < n_out; ++i) {
        for (const Range &r : r_in)
            if (overlaps(r_out[i], r))
                return MAMBA_ERR_ALIASING;
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(r_out[i], r_out[j]))
                return MAMBA_ERR_ALIASING;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (!has_seq) {
        // nothing ran: dh0 = dh_last, the parameters' and the look-back's gradients zero
        hipError_t e = hipSuccess;
        if (dh0)
            e = launch_copy_state(dh0, dh_last, bdn, st);
        if (e == hipSuccess && dA)
            e = launch_copy_state(dA, nullptr, dn, st);
        if (e == hipSuccess && dD)
            e = launch_copy_state(dD, nullptr, d_inner, st);
        if (e == hipSuccess && d_delta_bias)
            e = launch_copy_state(d_delta_bias, nullptr, d_inner, st);
        // (zero fills: rows of no source entries padded to one entry of 0)
        if (e == hipSuccess && du_prev)
            e = launch_pad_rows(du_prev, nullptr, bd, 0, 1, (int32_t)es, 0.0f, st);
        if (e == hipSuccess && dB_prev)
            e = launch_pad_rows(dB_prev, nullptr, bn, 0, 1, (int32_t)es, 0.0f, st);
        return hip_status(e);
    }
    char *ws = static_cast<char *>(workspace);
    M3BwdLaunch q{};
    q.u = u;
    q.delta = delta;
    q.z = z;
    q.dy = dy;
    q.B = B;
    q.C = C;
    q.lam = lam;
    q.u_prev = u_prev;
    q.B_prev = B_prev;
    q.theta = theta;
    q.A = A;
    q.D = D;
    q.bias = delta_bias;
    q.h0 = h0;
    q.dh_last = dh_last;
    q.du = du;
    q.ddelta = ddelta;
    q.dz = dz;
    q.dB = dB;
    q.dC = dC;
    q.dlam = dlam;
    q.du_prev = du_prev;
    q.dB_prev = dB_prev;
    q.dtheta = dtheta;
    q.dA = dA;
    q.dD = dD;
    q.dbias = d_delta_bias;
    q.dh0 = dh0;
    auto region = [&](int i) { return reinterpret_cast<float *>(ws + off[i]); };
    q.ckpt = region(0);
    q.part = region(1);
    q.bprev_part = region(2);
    q.dA_part = region(3);
    q.dDb_part = region(4);
    q.batch = batch;
    q.L = seqlen;
    q.d_inner = d_inner;
    q.d_state = d_state;
    q.dtype = dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32;
    q.zoh = zoh;
    q.n_spans = plan.n_spans;
    q.span_len = plan.span_len;
    if (plan.n_spans > 1) {
        // the forward span pass over every span (its transitions also serve the adjoint
        // carry) and the carry: the state entering each span
        ScanLaunch E{};
        E.u = u;
        E.delta = delta;
        E.B = B;
        E.C = C;
        E.A = A;
        E.bias = delta_bias;
        E.lam = lam;
        E.u_prev = u_prev;
        E.B_prev = B_prev;
        E.theta = theta;
        E.trap = lam != nullptr;
        E.rot = theta != nullptr;
        E.zoh = zoh;
        E.ws_decay = region(6);
        E.ws_hloc = region(7);
        E.ws_rot = theta ? region(9) : nullptr;
        E.batch = batch;
        E.L = seqlen;
        E.d_inner = d_inner;
        E.d_state = d_state;
        E.span_len = plan.span_len;
        E.n_spans = plan.n_spans;
        E.first_span = 0;
        E.launch_spans = plan.n_spans;
        E.waves = plan.fwd_waves;
        E.chunk = plan.fwd_chunk;
        E.dtype = q.dtype;
        E.bc_staged = region(5);
        E.staged_rows = seqlen + plan.fwd_chunk;
        E.relay_parts = 1;
        E.su = E.sd = E.sz = d_inner;
        E.sB = E.sC = d_state;
        if (launch_stage_bc(E, st) != hipSuccess || launch_scalar_end(E, st) != hipSuccess)
            return MAMBA_ERR_HIP;
        CarryLaunch K{};
        K.ws_decay = region(6);
        K.ws_hloc = region(7);
        K.ws_rot = theta ? region(9) : nullptr;
        K.h0 = h0;
        K.h_in = region(8);
        K.columns = batch * d_inner * d_state;
        K.n_spans = plan.n_spans;
        if (launch_carry(K, st) != hipSuccess)
            return MAMBA_ERR_HIP;
        q.ws_decay = region(6);
        q.ws_rot = theta ? region(9) : nullptr;
        q.h_in = region(8);
        q.mu_loc = region(10);
        q.mu_in = region(11);
        q.du_edge = region(12);
        q.du_lb = region(13);
    }
    return hip_status(launch_scan_bwd_m3(q, st));
}

mamba_status_t mamba_scan_bwd_ckpt(const void *u, const void *delta, const float *A,
                                   const void *B, const void *C, const float *D, const void *z,
                                   const float *delta_bias, const float *h0, const void *dy,
                                   const float *dh_last, const float *ckpt, void *du,
                                   void *ddelta, float *dA, void *dB, void *dC, float *dD,
                                   void *dz, float *d_delta_bias, float *dh0, int64_t batch,
                                   int64_t seqlen, int64_t d_inner, int64_t d_state,
                                   mamba_dtype_t dtype, void *workspace, size_t workspace_bytes,
                                   const mamba_scan_opts_t *opts, void *stream)
{
    if (!ckpt && seqlen > 0)
        return MAMBA_ERR_NULL_ARG;
    return bwd_impl(u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_last,
                    seqlen > 0 ? ckpt : nullptr, du, ddelta, dA, dB, dC, dD, dz, d_delta_bias,
                    dh0, batch, seqlen, d_inner, d_state, dtype, workspace, workspace_bytes, opts,
                    stream);
}


int32_t mamba_ssd_supported(int64_t head_dim, int64_t d_state)
{
    return ssd_supported(head_dim, d_state) ? 1 : 0;
}

// SSD launch plan (mamba_ssd_fwd_ex): a sequence split into spans when the units are too few
// for the device, else the relay of a partial last round (the second parts from step
// relay_mid, whole chunks before it).
struct SsdPlan {
    int64_t relay_units = 0, relay_mid = 0;
    bool relay_withhold = false; // failure test (relay = -2): part 0 keeps its state
    int64_t n_spans = 1, span_len = 0;
};

static mamba_status_t ssd_check_shape(int64_t batch, int64_t seqlen, int64_t n_heads,
                                      int64_t head_dim, int64_t d_state, mamba_dtype_t dtype)
{
    if (batch < 0 || seqlen < 0 || n_heads < 0 || head_dim <= 0 || d_state <= 0)
        return MAMBA_ERR_BAD_SHAPE;
    if (dtype != MAMBA_DTYPE_F32 && dtype != MAMBA_DTYPE_BF16)
        return MAMBA_ERR_BAD_DTYPE;
    if (!ssd_supported(head_dim, d_state))
        return MAMBA_ERR_UNSUPPORTED;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    int64_t dn, bld, blh, bln, bdn, t;
    if (!mul_ok(n_heads, head_dim, &dn) || !mul_ok(batch, seqlen, &t) ||
        !mul_ok(t, dn, &bld) || !mul_ok(bld, es, &t) || !mul_ok(batch * seqlen, n_heads, &blh) ||
        !mul_ok(blh, es, &t) || !mul_ok(batch * seqlen, d_state, &bln) || !mul_ok(bln, es, &t) ||
        !mul_ok(batch, dn, &t) || !mul_ok(t, d_state, &bdn) || !mul_ok(bdn, 4, &t) ||
        dn > INT32_MAX || batch * n_heads > INT32_MAX)
        return MAMBA_ERR_BAD_SHAPE;
    if (dn * es * 64 > INT32_MAX) // a chunk of 64 rows is addressed with 32-bit offsets
        return MAMBA_ERR_UNSUPPORTED;
    return MAMBA_OK;
}

// (shapes already checked)
static mamba_status_t ssd_make_plan(int64_t batch, int64_t seqlen, int64_t n_heads,
                                    int64_t d_state, mamba_dtype_t dtype,
                                    const mamba_ssd_opts_t *opts, SsdPlan *r)
{
    *r = SsdPlan{};
    int32_t relay = opts ? opts->relay : 0;
    const int32_t spans = opts ? opts->n_spans : 0;
    if (relay == -2) { // forced relay whose first parts withhold their hand-off (testing)
        r->relay_withhold = true;
        relay = 2;
    }
    if (relay < 0 || relay > 2 || spans < 0 || spans > 64 || (relay == 2 && spans >= 2))
        return MAMBA_ERR_UNSUPPORTED;
    const int64_t units = batch * n_heads;
    const int64_t chunks = (seqlen + 63) / 64;
    if (units <= 0 || chunks < 2)
        return MAMBA_OK;
    const int64_t slots =
        ssd_block_slots(d_state, dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32);

    // Split: as many spans as fill one round of the slots, of at least 8 chunks each.
    int64_t k = 1;
    if (spans >= 2)
        k = spans;
    else if (spans == 0 && relay != 2 && slots > 0 && 2 * units <= slots)
        k = std::min(slots / units, chunks / 8);
    if (k >= 2) {
        const int64_t per = (chunks + k - 1) / k; // chunks per span
        k = (chunks + per - 1) / per;             // every span non-empty
        if (k >= 2 && units * k <= INT32_MAX) {
            r->n_spans = k;
            r->span_len = per * 64;
            return MAMBA_OK;
        }
    }
    if (relay == 1)
        return MAMBA_OK;
    int64_t rem = slots > 0 ? units % slots : 0;
    if (relay == 2) {
        if (rem == 0)
            rem = units;
    } else if (!(slots > 0 && units > slots && rem > 0 && 2 * rem <= slots && chunks >= 8)) {
        return MAMBA_OK;
    }
    if (rem > INT32_MAX - units) // the grid holds units + rem blocks
        return MAMBA_OK;
    r->relay_units = rem;
    r->relay_mid = (chunks + 1) / 2 * 64;
    return MAMBA_OK;
}

// Workspace: relay [one flag per relayed unit and a fault word, 256-byte aligned][head_dim x
// d_state fp32 each]; split [(n_spans - 1) x units states of head_dim x d_state fp32]
// [(n_spans - 1) x units decays, fp32].
static size_t ssd_sync_bytes(const SsdPlan &r)
{
    return r.relay_units > 0
               ? (((size_t)r.relay_units + 1) * sizeof(uint32_t) + 255) / 256 * 256
               : 0;
}

static size_t ssd_span_state_bytes(const SsdPlan &r, int64_t units, int64_t head_dim,
                                   int64_t d_state)
{
    if (r.n_spans < 2)
        return 0;
    return (size_t)(r.n_spans - 1) * (size_t)units * (size_t)head_dim * (size_t)d_state *
           sizeof(float);
}

static size_t ssd_workspace_bytes(const SsdPlan &r, int64_t units, int64_t head_dim,
                                  int64_t d_state)
{
    if (r.n_spans >= 2)
        return ssd_span_state_bytes(r, units, head_dim, d_state) +
               (size_t)(r.n_spans - 1) * (size_t)units * sizeof(float);
    if (r.relay_units <= 0)
        return 0;
    return ssd_sync_bytes(r) +
           (size_t)r.relay_units * (size_t)head_dim * (size_t)d_state * sizeof(float);
}

size_t mamba_ssd_workspace_size(int64_t batch, int64_t seqlen, int64_t n_heads,
                                int64_t head_dim, int64_t d_state, mamba_dtype_t dtype,
                                const mamba_ssd_opts_t *opts)
{
    SsdPlan r;
    if (ssd_check_shape(batch, seqlen, n_heads, head_dim, d_state, dtype) != MAMBA_OK ||
        ssd_make_plan(batch, seqlen, n_heads, d_state, dtype, opts, &r) != MAMBA_OK)
        return (size_t)-1;
    return ssd_workspace_bytes(r, batch * n_heads, head_dim, d_state);
}

mamba_status_t mamba_ssd_fwd_ex(const void *x, const void *dt, const float *A, const void *B,
                                const void *C, const float *D, const void *z,
                                const float *dt_bias, const float *h0, void *y, float *h_last,
                                int64_t batch, int64_t seqlen, int64_t n_heads,
                                int64_t head_dim, int64_t d_state, mamba_dtype_t dtype,
                                void *workspace, size_t workspace_bytes,
                                const mamba_ssd_opts_t *opts, void *stream)
{
    const mamba_status_t shape_st =
        ssd_check_shape(batch, seqlen, n_heads, head_dim, d_state, dtype);
    if (shape_st != MAMBA_OK)
        return shape_st;
    SsdPlan plan;
    const mamba_status_t plan_st =
        ssd_make_plan(batch, seqlen, n_heads, d_state, dtype, opts, &plan);
    if (plan_st != MAMBA_OK)
        return plan_st;
    if (batch == 0 || n_heads == 0)
        return MAMBA_OK;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    const int64_t dn = n_heads * head_dim;
    const int64_t bld = batch * seqlen * dn, blh = batch * seqlen * n_heads;
    const int64_t bln = batch * seqlen * d_state, bdn = batch * dn * d_state;
    const bool has_seq = seqlen > 0;
    if (!A || (has_seq && (!x || !dt || !B || !C || !y)))
        return MAMBA_ERR_NULL_ARG;
    const void *elem_ptrs[] = {dt, y};
    for (const void *p : elem_ptrs)
        if (p && !aligned(p, (size_t)es))
            return MAMBA_ERR_MISALIGNED;
    const void *vec_ptrs[] = {x, B, C, z}; // read as 16-byte vectors
    for (const void *p : vec_ptrs)
        if (p && !aligned(p, 16))
            return MAMBA_ERR_MISALIGNED;
    const void *f32_ptrs[] = {A, D, dt_bias, h0, h_last};
    for (const void *p : f32_ptrs)
        if (p && !aligned(p, 4))
            return MAMBA_ERR_MISALIGNED;
    const size_t need = ssd_workspace_bytes(plan, batch * n_heads, head_dim, d_state);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return MAMBA_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 4))
        return MAMBA_ERR_MISALIGNED;
    const Range r_in[] = {range_of(x, bld * es),         range_of(dt, blh * es),
                          range_of(B, bln * es),         range_of(C, bln * es),
                          range_of(z, bld * es),         range_of(A, n_heads * 4),
                          range_of(D, n_heads * 4),      range_of(dt_bias, n_heads * 4)};
    const Range r_h0 = range_of(h0, bdn * 4);
    const Range r_y = range_of(has_seq ? y : nullptr, bld * es);
    const Range r_hl = range_of(h_last, bdn * 4);
    const Range r_ws = range_of(need > 0 ? workspace : nullptr, (int64_t)need);
    for (const Range &r : r_in)
        if (overlaps(r_y, r) || overlaps(r_hl, r) || overlaps(r_ws, r))
            return MAMBA_ERR_ALIASING;
    if (overlaps(r_y, r_h0) || overlaps(r_y, r_hl) || overlaps(r_hl, r_h0))
        return MAMBA_ERR_ALIASING; // (h_last is written while h0 is still being read)
    if (overlaps(r_ws, r_h0) || overlaps(r_ws, r_y) || overlaps(r_ws, r_hl))
        return MAMBA_ERR_ALIASING;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (!has_seq) {
        if (h_last)
            return hip_status(launch_copy_state(h_last, h0, bdn, st));
        return MAMBA_OK;
    }
    SsdLaunch q{};
    q.x = x;
    q.dt = dt;
    q.B = B;
    q.C = C;
    q.z = z;
    q.A = A;
    q.D = D;
    q.dt_bias = dt_bias;
    q.h0 = h0;
    q.y = y;
    q.h_last = h_last;
    q.batch = batch;
    q.L = seqlen;
    q.n_heads = n_heads;
    q.head_dim = head_dim;
    q.d_state = d_state;
    q.dtype = dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32;
    char *ws = static_cast<char *>(workspace);
    if (plan.n_spans >= 2) {
        q.n_spans = plan.n_spans;
        q.span_len = plan.span_len;
        q.span_state = reinterpret_cast<float *>(ws);
        q.span_decay = reinterpret_cast<float *>(
            ws + ssd_span_state_bytes(plan, batch * n_heads, head_dim, d_state));
    } else if (plan.relay_units > 0) {
        q.relay_units = plan.relay_units;
        q.relay_mid = plan.relay_mid;
        q.relay_sync = reinterpret_cast<uint32_t *>(ws);
        q.relay_state = reinterpret_cast<float *>(ws + ssd_sync_bytes(plan));
        q.relay_withhold = plan.relay_withhold;
    }
    return hip_status(launch_ssd(q, st));
}

mamba_status_t mamba_ssd_relay_faults(const void *workspace, size_t workspace_bytes,
                                      int64_t batch, int64_t seqlen, int64_t n_heads,
                                      int64_t head_dim, int64_t d_state, mamba_dtype_t dtype,
                                      const mamba_ssd_opts_t *opts, uint32_t *faults,
                                      void *stream)
{
    if (!faults)
        return MAMBA_ERR_NULL_ARG;
    *faults = 0;
    const mamba_status_t shape_st =
        ssd_check_shape(batch, seqlen, n_heads, head_dim, d_state, dtype);
    if (shape_st != MAMBA_OK)
        return shape_st;
    SsdPlan plan;
    const mamba_status_t plan_st =
        ssd_make_plan(batch, seqlen, n_heads, d_state, dtype, opts, &plan);
    if (plan_st != MAMBA_OK)
        return plan_st;
    if (plan.n_spans >= 2 || plan.relay_units <= 0 || batch == 0 || n_heads == 0 || seqlen == 0)
        return MAMBA_OK; // no relay: nothing can have timed out
    const size_t need = ssd_workspace_bytes(plan, batch * n_heads, head_dim, d_state);
    if (!workspace || workspace_bytes < need)
        return MAMBA_ERR_WORKSPACE;
    return read_fault_word(static_cast<const uint32_t *>(workspace) + plan.relay_units, faults,
                           stream);
}

mamba_status_t mamba_ssd_state_update(float *h, const void *x, const void *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const void *z, const float *dt_bias, void *y,
                                      int64_t batch, int64_t n_heads, int64_t head_dim,
                                      int64_t d_state, mamba_dtype_t dtype, void *stream)
{
    const mamba_status_t shape_st = ssd_check_shape(batch, 1, n_heads, head_dim, d_state, dtype);
    if (shape_st != MAMBA_OK)
        return shape_st;
    if (batch == 0 || n_heads == 0)
        return MAMBA_OK;
    if (!h || !x || !dt || !A || !B || !C || !y)
        return MAMBA_ERR_NULL_ARG;
    const int64_t es = dtype == MAMBA_DTYPE_F32 ? 4 : 2;
    const int64_t dn = n_heads * head_dim, bd = batch * dn, bh = batch * n_heads;
    const int64_t bn = batch * d_state, bdn = bd * d_state;
    const void *elem_ptrs[] = {x, dt, B, C, z, y};
    for (const void *p : elem_ptrs)
        if (p && !aligned(p, (size_t)es))
            return MAMBA_ERR_MISALIGNED;
    const void *f32_ptrs[] = {A, D, dt_bias};
    for (const void *p : f32_ptrs)
        if (p && !aligned(p, 4))
            return MAMBA_ERR_MISALIGNED;
    if (!aligned(h, 16)) // moved as 16-byte vectors
        return MAMBA_ERR_MISALIGNED;
    const Range r_in[] = {range_of(x, bd * es),          range_of(dt, bh * es),
                          range_of(z, bd * es),          range_of(B, bn * es),
                          range_of(C, bn * es),          range_of(A, n_heads * 4),
                          range_of(D, n_heads * 4),      range_of(dt_bias, n_heads * 4)};
    const Range r_h = range_of(h, bdn * 4);
    const Range r_y = range_of(y, bd * es);
    if (overlaps(r_h, r_y))
        return MAMBA_ERR_ALIASING;
    for (const Range &r : r_in)
        if (overlaps(r_h, r) || overlaps(r_y, r))
            return MAMBA_ERR_ALIASING;
    SsdStepLaunch S{};
    S.h = h;
    S.x = x;
    S.dt = dt;
    S.B = B;
    S.C = C;
    S.z = z;
    S.A = A;
    S.D = D;
    S.dt_bias = dt_bias;
    S.y = y;
    S.batch = batch;
    S.n_heads = n_heads;
    S.head_dim = head_dim;
    S.d_state = d_state;
    S.dtype = dtype == MAMBA_DTYPE_BF16 ? DType::BF16 : DType::F32;
    return hip_status(launch_ssd_step(S, reinterpret_cast<hipStream_t>(stream)));
}

mamba_status_t mamba_ssd_fwd(const void *x, const void *dt, const float *A, const void *B,
                             const void *C, const float *D, const void *z,
                             const float *dt_bias, const float *h0, void *y, float *h_last,
                             int64_t batch, int64_t seqlen, int64_t n_heads, int64_t head_dim,
                             int64_t d_state, mamba_dtype_t dtype, void *stream)
{
    const mamba_ssd_opts_t plain = {1, 1}; // no relay, no split
    return mamba_ssd_fwd_ex(x, dt, A, B, C, D, z, dt_bias, h0, y, h_last, batch, seqlen,
                            n_heads, head_dim, d_state, dtype, nullptr, 0, &plain, stream);
}

} // extern "C"
