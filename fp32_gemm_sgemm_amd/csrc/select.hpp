// Variant description and the shape-aware selector: pure host logic, no HIP
// calls, so it can be exercised without a device.
//
// Geometry uses round-up-and-guard sizing (DD2360 workbook "Applied GPU
// Programming", Module 6, section 6.3): tiles_m = ceil(M/BM),
// tiles_n = ceil(N/BN), one workgroup per tile, K split and batch entry.
// The selector weighs per-tile efficiency against wave quantisation: on S
// compute units a grid of n equal workgroups takes ceil(n/S) rounds ("4.1
// CUDA GEMM operator performance optimization", section 12.5 on launching at
// least as many blocks as SMs and tuning per shape; the workbook's Module 17
// on the tail effect).  When a grid has too few tiles, splitting K across
// workgroups adds rounds' worth of parallel work at the price of a second,
// memory-bound pass that adds the partial results (the split-K stage of the
// "cuda-kernels" README).
#pragma once

#include <limits.h>
#include <stdint.h>

#include "sgemm.h"

namespace sgemm {

struct Variant {
    int kernel;
    int bm, bn, bk;
    int waves_m, waves_n;
    int stage_at;      // register-staged kernel: LDS write after this k group
    int stages;        // direct-load kernel: LDS stages (0 = register-staged kernel)
    int dword;         // direct-load kernel with 4-byte loads (for rows not 16-byte aligned)
    int threads;
    int lds_bytes;
    const void *fn[4];  // kernel per operand layout, index transa + 2*transb (null: none)
    int eff_permille;   // measured steady-state fraction of the FP32 matrix peak
                        // (x1000; the FP32 vector-FMA peak is the same figure) over
                        // rounds of full tiles; 0 = never chosen by the selector
    int eff_one_permille;        // the same when the grid has at most one workgroup
                                 // per CU (no co-resident workgroups to hide latency)
    int eff_unaligned_permille;  // the same as eff_permille when rows are not
                                 // 16-byte aligned (4-byte direct loads for the variants
                                 // that have them, every slice fetched through registers
                                 // for the other direct-load ones)
    int fixed_ns;                // fixed cost of a tile in the cost model (0: kTileFixedNs)
    int spill_permille;          // slice cost (x1000 of the resident one) once the operand
                                 // rows and columns the tiles of one XCD read exceed its
                                 // L2, over one round (0: not modelled)
    int spill_full_permille;     // the same over several rounds, where every CU streams
                                 // (0: not modelled)
    int coresident;              // workgroups that share a CU and overlap their fixed
                                 // costs (0: one, the fixed cost is paid every round)
    int ld64;                    // addresses its operands in 64 bits throughout: any
                                 // leading dimension (0: the tile limits below apply)
};

// One call as the planner sees it.
struct Problem {
    int transa, transb;
    int M, N, K;
    int lda, ldb, ldc;
    int batch;
};

inline int op_index(const Problem &p) { return p.transa + 2 * p.transb; }

// Largest sizes accepted (k0 + BK and similar sums stay in int); leading
// dimensions up to the same.
constexpr int kMaxDim = INT_MAX - 1024;
// Leading dimensions the LDS-tiled kernels serve: the byte offsets of a
// thread inside one slice stay below 2^32, for up to 256 rows of a
// k-contiguous operand (A, or a transposed B) and 32 rows of an
// index-contiguous one (B, or a transposed A).  Beyond them the selector
// keeps to the variants that address in 64 bits (ld64: the 32 x 32, 16 x 16
// and 8 x 8 tiles that split K inside the workgroup) and to the strip kernel.
constexpr int kMaxLdK = (1 << 22) - 64;
constexpr int kMaxLdX = (1 << 25) - 512;
// Direct global -> LDS loads keep those offsets below 2^31 (the offset given
// to chunks that must read as zero).
constexpr int kMaxLdKDirect = 1 << 20;
constexpr int kMaxLdXDirect = 1 << 24;
// Variants with 64-deep slices hold 64 rows of an index-contiguous operand,
// so they serve only leading dimensions up to this (offsets below 2^31 on
// every fetch path).
constexpr int kMaxLdXDeep = 1 << 23;

// Whether variant v can serve problem p (beyond the sizes every variant takes).
inline bool variant_fits(const Variant &v, const Problem &p)
{
    if (v.ld64) return true;
    if (p.lda > (p.transa ? kMaxLdX : kMaxLdK) || p.ldb > (p.transb ? kMaxLdK : kMaxLdX))
        return false;
    if (v.bk <= 32) return true;
    const int ldx_a = p.transa ? p.lda : 0, ldx_b = p.transb ? 0 : p.ldb;
    return ldx_a <= kMaxLdXDeep && ldx_b <= kMaxLdXDeep;
}

inline bool sizes_ok(const Problem &p)
{
    if (p.transa < 0 || p.transa > 1 || p.transb < 0 || p.transb > 1) return false;
    if (p.M < 0 || p.N < 0 || p.K < 0 || p.batch < 0) return false;
    if (p.M > kMaxDim || p.N > kMaxDim || p.K > kMaxDim) return false;
    const int a_min = p.transa ? p.M : p.K, b_min = p.transb ? p.K : p.N;
    if (p.lda < (a_min > 1 ? a_min : 1) || p.ldb < (b_min > 1 ? b_min : 1) ||
        p.ldc < (p.N > 1 ? p.N : 1))
        return false;
    return p.lda <= kMaxDim && p.ldb <= kMaxDim && p.ldc <= kMaxDim;
}

inline bool direct_lds_ok(const Problem &p)
{
    return p.lda <= (p.transa ? kMaxLdXDirect : kMaxLdKDirect) &&
           p.ldb <= (p.transb ? kMaxLdKDirect : kMaxLdXDirect);
}

inline long long ceil_div_ll(long long a, long long b) { return (a + b - 1) / b; }

// K per split is a multiple of this: of every variant's slice depth (and of
// the register-staged kernel's slice pairs).
constexpr int kSplitAlign = 64;
constexpr int kMaxSplits = 64;

// Split count and K range of one split for a requested split count.
inline void split_k(int K, int want, int &splits, int &k_chunk)
{
    if (want <= 1 || K <= kSplitAlign) {
        splits = 1;
        k_chunk = K > 0 ? K : 1;
        return;
    }
    if (want > kMaxSplits) want = kMaxSplits;
    const long long per = ceil_div_ll(K, want);
    k_chunk = (int)(ceil_div_ll(per, kSplitAlign) * kSplitAlign);
    splits = (int)ceil_div_ll(K, k_chunk);
    if (splits <= 1) k_chunk = K;
}

// Edge strips: at most this many rows (or columns) of C go to the strip
// kernel instead of a row (or column) of tiles.
constexpr int kStripMaxWidth = 4;

// The block the tiled kernel computes when sm rows and sn columns of C go to
// strips: the first M - sm rows and N - sn columns.
inline Problem main_block(const Problem &p, int sm, int sn)
{
    Problem q = p;
    q.M = p.M - sm;
    q.N = p.N - sn;
    return q;
}

// Row stride of the partial results (16-byte rows).
inline long long partial_ld(int N) { return ((long long)N + 3) & ~3ll; }

inline long long split_workspace_bytes(const Problem &p, int splits)
{
    if (splits <= 1) return 0;
    return (long long)p.batch * splits * p.M * partial_ld(p.N) * 4;
}

// Fixed cost of one tile (prologue fetch, pipeline fill, epilogue stores) for
// the variants that do not carry their own.
constexpr double kTileFixedNs = 2500.0;

inline void describe(const Variant &v, int id, sgemm_cfg *out)
{
    out->id = id;
    out->kernel = v.kernel;
    out->bm = v.bm;
    out->bn = v.bn;
    out->bk = v.bk;
    out->waves_m = v.waves_m;
    out->waves_n = v.waves_n;
    out->group_m = 0;
    out->xcd_remap = 0;
    out->splits = 1;
    out->k_chunk = 0;
    out->grid = 0;
    out->threads = v.threads;
    out->lds_bytes = v.lds_bytes;
    out->tiles_m = 0;
    out->tiles_n = 0;
    out->workspace_bytes = 0;
    out->strip_m = 0;
    out->strip_n = 0;
    out->fixed_ns = v.fixed_ns > 0 ? v.fixed_ns : (int)kTileFixedNs;
    out->spill_permille = v.spill_permille;
    out->spill_full_permille = v.spill_full_permille;
    out->coresident = v.coresident > 1 ? v.coresident : 1;
}

// Default tile order: groups of 8 tile rows and the XCD remap.
constexpr int kDefaultGroupM = 8;
constexpr int kDefaultXcdRemap = 1;

// Whether sm rows and sn columns of C may go to strips.
inline bool strips_ok(const Problem &p, int sm, int sn)
{
    return sm >= 0 && sn >= 0 && sm <= kStripMaxWidth && sn <= kStripMaxWidth && sm <= p.M &&
           sn <= p.N;
}

// Fills the geometry of variant v with `want` K splits for the block left
// after sm rows and sn columns go to strips (the tile counts, grid, split and
// workspace describe that block; an empty block has grid 0); false if the
// grid does not fit in an int or the strips are out of range.
inline bool finish_cfg(const Variant &v, int id, const Problem &full, int want, int sm, int sn,
                       sgemm_cfg *out)
{
    if (!strips_ok(full, sm, sn)) return false;
    const Problem p = main_block(full, sm, sn);
    describe(v, id, out);
    out->strip_m = sm;
    out->strip_n = sn;
    if (p.M == 0 || p.N == 0) want = 1;  // no tiled block: nothing to split
    int splits, k_chunk;
    split_k(p.K, want, splits, k_chunk);
    const long long tm = ceil_div_ll(p.M, v.bm), tn = ceil_div_ll(p.N, v.bn);
    const long long grid = tm * tn * splits * (long long)p.batch;
    if (tm * tn > INT_MAX || grid > INT_MAX) return false;
    out->tiles_m = (int)tm;
    out->tiles_n = (int)tn;
    out->grid = (int)grid;
    out->splits = splits;
    out->k_chunk = k_chunk;
    out->workspace_bytes = split_workspace_bytes(p, splits);
    out->group_m = kDefaultGroupM;
    out->xcd_remap = kDefaultXcdRemap;
    return true;
}

// ---- cost model (nanoseconds) ---------------------------------------------------
// One compute unit at the FP32 matrix peak: 157.3 TFLOP/s over 256 CUs.
constexpr double kCuFlopPerNs = 157.3e3 / 256.0;
// The reduction pass: the second launch and the wait for the first one to
// drain (a split product measured 7-10 us above its main kernel's model at
// 512^3 and 128 x 128 x 32768), and the rate at which it streams the
// partials and writes C (about 5 TB/s).
constexpr double kReduceFixedNs = 7500.0;
constexpr double kReduceBytesPerNs = 5000.0;

// L2 per XCD, and the XCDs of the chip.  Operands count as held in L2 up to
// 15/16 of it (the rest holds C and whatever else passes through): a round of
// 64 x 64 tiles slows past 3.8-3.9 MiB of operand rows and columns per XCD
// (1024 x 1024 x K, K = 1280 to 1344, measured on MI355X).
constexpr double kL2Bytes = 4.0 * 1024 * 1024;
constexpr double kL2OperandBytes = kL2Bytes * 15.0 / 16.0;
constexpr int kXcds = 8;

// Bytes of op(A) rows and op(B) columns, over kc values of k, that the tiles
// one XCD runs in the first round read, for the XCD that reads the most.  It
// follows the launch order of the kernels (common.hpp xcd_order and work_of,
// with groups of kDefaultGroupM tile rows): each XCD takes a contiguous run of
// logical tile ids, which walks a group of tile rows column by column, and a
// run that crosses into the next group (or the next K split or batch entry,
// whose operands differ) reads the rows and columns of both.
inline double xcd_operand_bytes(const Variant &v, long long tiles_m, long long tiles_n,
                                long long grid, int kc, int cus)
{
    const long long mn = tiles_m * tiles_n;
    const long long per_group = kDefaultGroupM * tiles_n;
    const long long q = grid / kXcds, r = grid % kXcds;
    const long long first_round = grid < cus ? grid : cus;
    double worst = 0.0;
    for (int x = 0; x < kXcds; ++x) {
        // hardware workgroups x, x + 8, ... of the first round; their logical
        // ids start at the XCD's block
        const long long n = first_round > x ? (first_round - 1 - x) / kXcds + 1 : 0;
        long long pos = x * q + (x < r ? x : r);
        const long long end = pos + n;
        long long rows = 0, cols = 0;
        while (pos < end) {
            const long long t = pos % mn;  // tile within its (split, batch) block
            const long long grp = t / per_group;
            const long long g_rows = tiles_m - grp * kDefaultGroupM < kDefaultGroupM
                                         ? tiles_m - grp * kDefaultGroupM
                                         : kDefaultGroupM;
            const long long a = t - grp * per_group;  // first index inside the group
            long long b = a + (end - pos);             // one past the last, capped at the group
            if (b > g_rows * tiles_n) b = g_rows * tiles_n;
            rows += b - a < g_rows ? b - a : g_rows;
            cols += (b - 1) / g_rows - a / g_rows + 1;
            pos += b - a;
        }
        const double bytes = 4.0 * kc * (double)(rows * v.bm + cols * v.bn);
        if (bytes > worst) worst = bytes;
    }
    return worst;
}

// eff: the variant's fraction of peak (x1000) for this call's alignment.
inline double estimate_ns(const Variant &v, const Problem &p, int splits, int k_chunk, int cus,
                          int eff)
{
    const long long tiles = ceil_div_ll(p.M, v.bm) * ceil_div_ll(p.N, v.bn) * splits * (long long)p.batch;
    const long long rounds = ceil_div_ll(tiles, cus);
    const int kc = splits > 1 ? k_chunk : p.K;
    long long slices = ceil_div_ll(kc, v.bk);
    if (v.stages == 0 && v.stage_at >= 0) slices += slices & 1;  // register pipeline takes pairs
    double e = eff;
    if (tiles <= cus) e = e * v.eff_one_permille / v.eff_permille;
    double slice_ns = 2.0 * v.bm * v.bn * v.bk / (kCuFlopPerNs * e / 1000.0);
    const int spill = tiles <= cus ? v.spill_permille : v.spill_full_permille;
    if (spill > 0 && xcd_operand_bytes(v, ceil_div_ll(p.M, v.bm), ceil_div_ll(p.N, v.bn), tiles, kc,
                                       cus) > kL2OperandBytes)
        slice_ns = slice_ns * spill / 1000.0;
    const double fixed = v.fixed_ns > 0 ? (double)v.fixed_ns : kTileFixedNs;
    // co-resident workgroups pay their fixed costs together, once per wave of
    // cus * coresident tiles, and share the CU's matrix cores for the slices
    const long long waves = v.coresident > 1 ? ceil_div_ll(tiles, (long long)cus * v.coresident)
                                             : rounds;
    double t = (double)waves * fixed + (double)rounds * (double)slices * slice_ns;
    if (splits > 1)
        t += kReduceFixedNs +
             4.0 * (double)p.batch * p.M * (double)partial_ld(p.N) * (splits + 1) / kReduceBytesPerNs;
    return t;
}

// ---- edge strips: geometry and cost ------------------------------------------
// x (the strip's long index) per strip workgroup: 32, or 16 for a KC strip
// (streamed rows along k) when the launch's strips have fewer workgroups than
// the CUs, which doubles their workgroups (measured 20-23% faster on
// 2048-row strips).  An XC strip keeps 32 (its 128-byte row segments).
constexpr int kStripWidth = 32;
constexpr int kStripNarrowWidth = 16;

struct StripShape {
    long long x;  // outputs along the strip (0: no strip)
    int wgs;      // workgroups per batch entry
    bool kc;      // the streamed operand's rows run along k
    bool narrow;  // 16 x per workgroup
};
struct StripPlan {
    StripShape row, col;  // rows M-sm.. of C (streams op(B)); columns N-sn.. of the rows above (op(A))
};

// The strips of a plan with sm rows and sn columns on `cus` compute units:
// what the launch runs and what the cost model prices.
inline StripPlan strip_plan(const Problem &p, int sm, int sn, int cus)
{
    StripPlan g = {};
    const long long m_main = (long long)p.M - sm;
    if (sm > 0) {
        g.row.x = p.N;
        g.row.kc = p.transb != 0;
        g.row.wgs = (int)ceil_div_ll(p.N, kStripWidth);
    }
    if (sn > 0 && m_main > 0) {
        g.col.x = m_main;
        g.col.kc = p.transa == 0;
        g.col.wgs = (int)ceil_div_ll(m_main, kStripWidth);
    }
    if (((long long)g.row.wgs + g.col.wgs) * p.batch < cus) {
        for (StripShape *s : {&g.row, &g.col}) {
            if (s->wgs && s->kc) {
                s->narrow = true;
                s->wgs = (int)ceil_div_ll(s->x, kStripNarrowWidth);
            }
        }
    }
    return g;
}

// The strip kernel's cost: one launch for both strips, each streaming the
// operand it reads whole (op(B) for the row strip, the first M - sm rows of
// op(A) for the column strip).  A strip streams at the chip's rate for its
// order once it has enough workgroups, and otherwise at a per-workgroup rate
// times its workgroups: a strip workgroup covers all of K, so a strip of few
// columns runs on few CUs ("4.1 CUDA GEMM operator performance optimization",
// section 12.5, on grids smaller than the SM count).  Fitted on MI355X by
// fp32_gemm_sgemm_amd.calibrate: strip-only products streaming op(B), the
// chip's rates from 256 and 512 workgroups, the per-workgroup rates from 8
// (XC) and 16 narrow (KC) workgroups with long K.
constexpr double kStripFixedNs = 7600.0;       // one launch, the launch floor included
constexpr double kStripBytesPerNs = 3775.0;    // streamed rows along k (KC), whole chip
constexpr double kStripBytesPerNsXc = 5556.0;  // streamed rows along the strip (XC), whole chip
constexpr double kStripWgBytesPerNsXc = 37.0;  // one XC workgroup
constexpr double kStripWgBytesPerNsKcNarrow = 30.8;  // one narrow KC workgroup
// The launch floor (dispatch, completion) inside kStripFixedNs: a strip
// launch beside a tiled block pays it on top of the tiles' launch; strips
// that are the whole product pay it as every plan does, so the model, which
// leaves the floor out of the tiles' costs, leaves it out there too.
constexpr double kLaunchFloorNs = 3300.0;

inline double strip_stream_ns(const StripShape &s, int K, int batch)
{
    if (s.wgs == 0) return 0.0;
    const double chip = s.kc ? kStripBytesPerNs : kStripBytesPerNsXc;
    // a 32-wide KC strip runs only when the launch fills the CUs
    const double per_wg = s.kc ? (s.narrow ? kStripWgBytesPerNsKcNarrow : chip) : kStripWgBytesPerNsXc;
    const double wgs = (double)s.wgs * batch;
    const double rate = per_wg * wgs < chip ? per_wg * wgs : chip;
    return 4.0 * K * (double)s.x * batch / rate;
}

inline double strip_ns(const Problem &p, int sm, int sn, int cus)
{
    const StripPlan g = strip_plan(p, sm, sn, cus);
    if (g.row.wgs == 0 && g.col.wgs == 0) return 0.0;
    return kStripFixedNs + strip_stream_ns(g.row, p.K, p.batch) + strip_stream_ns(g.col, p.K, p.batch);
}

struct Choice {
    int id;
    int splits;
    int strip_m, strip_n;
};

// Candidate split counts tried by the selector.
constexpr int kSplitCandidates[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32, 48, 64};

// The efficiency (x1000) variant v is expected to reach on this call, or 0 if
// it does not apply.  aligned16: rows start 16-byte aligned; lds_ok: the
// leading dimensions allow direct-load offsets.  Strict (first pass): 16-byte
// direct-load variants only on aligned rows, 4-byte ones only on unaligned
// rows; otherwise (second pass) any variant, fetching through registers where
// direct loads do not apply.
inline int variant_eff(const Variant &v, bool aligned16, bool lds_ok, bool strict)
{
    if (v.stages == 0) return aligned16 ? v.eff_permille : v.eff_unaligned_permille;
    if (v.dword) {
        if (strict && (aligned16 || !lds_ok)) return 0;
        return v.eff_unaligned_permille;
    }
    if (strict && !(aligned16 && lds_ok)) return 0;
    return aligned16 && lds_ok ? v.eff_permille : v.eff_unaligned_permille;
}

// A 16-byte direct-load tile at the edge of an index-contiguous operand (B
// as stored, or A transposed) whose last 16-byte chunk is only partly inside
// N (or M) fetches every slice through registers, and the round waits for
// it: such a block is priced at the variant's unaligned rate (measured with
// every slice fetched through registers).
inline bool edge_chunks(const Variant &v, const Problem &q)
{
    if (v.stages == 0 || v.dword) return false;
    return (!q.transb && q.N % 4 != 0 && q.N % v.bn != 0) ||
           (q.transa && q.M % 4 != 0 && q.M % v.bm != 0);
}

// Strip widths worth trying along a dimension of size d with tile size b:
// none, and the rows past the last full tile when there are at most
// kStripMaxWidth of them (all of d when d itself is that small).
inline int strip_candidates(int d, int b, int (&out)[2])
{
    out[0] = 0;
    const int rem = d % b;
    if (rem >= 1 && rem <= kStripMaxWidth) {
        out[1] = rem;
        return 2;
    }
    return 1;
}

// The 8 x 8 vector-FMA tiles compete only from this K on, and not for
// products of at most kStripMaxWidth rows or columns.  Below that K a call is
// mostly fixed costs (theirs include a butterfly reduction across the wave),
// which their one fixed-cost figure prices poorly once several share a CU:
// measured on MI355X against the 16 x 16 tiles they would replace, 0.99-1.12
// of the time (geometric mean by K) for K = 256-2048, 0.70-0.87 for K = 4096-
// 65536.  Products of a few rows or columns waste most of an 8-row tile, and
// against the strip kernel they took up to 1.5 times as long.
constexpr int kVskMinK = 4096;

// Whether block q can split K across workgroups within `workspace_bytes`.
inline bool can_split(const Problem &q, long long workspace_bytes)
{
    int splits, k_chunk;
    split_k(q.K, 2, splits, k_chunk);
    return splits > 1 && split_workspace_bytes(q, splits) <= workspace_bytes;
}

// The fastest (variant, split count, strips) by the cost model among the
// variants compiled for the operand layout whose workspace fits in
// `workspace_bytes`.  Returns id -1 if no variant serves the layout.
// Tiles smaller than 32 x 32 (the 16 x 16 and 8 x 8 K-split ones) compete
// only where K cannot be split across workgroups: they read two and four
// times the operand bytes per flop of the 32 x 32 tiles, their rate depends
// on how many compute units stream at once (which the model does not
// capture), and with a workspace a split over larger tiles reaches the same
// parallelism with fewer bytes.
inline Choice select_plan(const Variant *vs, int n, const Problem &p, int cus, bool aligned16,
                          bool lds_ok, long long workspace_bytes)
{
    const int op = op_index(p);
    Choice best = {-1, 1, 0, 0};
    double best_t = 0;
    for (int pass = 0; pass < 2 && best.id < 0; ++pass) {
        for (int i = 0; i < n; ++i) {
            const Variant &v = vs[i];
            if (v.eff_permille <= 0 || v.eff_one_permille <= 0 ||
                v.eff_unaligned_permille <= 0 || !v.fn[op] || !variant_fits(v, p))
                continue;
            const int eff = variant_eff(v, aligned16, lds_ok, pass == 0);
            if (eff <= 0) continue;
            int sms[2], sns[2];
            const int nsm = strip_candidates(p.M, v.bm, sms), nsn = strip_candidates(p.N, v.bn, sns);
            for (int a = 0; a < nsm; ++a) {
                for (int b = 0; b < nsn; ++b) {
                    const Problem q = main_block(p, sms[a], sns[b]);
                    if (v.bm < 32 && q.M > 0 && q.N > 0 && can_split(q, workspace_bytes)) continue;
                    if (v.kernel == SGEMM_KERNEL_VALU &&
                        (q.K < kVskMinK || p.M <= kStripMaxWidth || p.N <= kStripMaxWidth))
                        continue;
                    double ts = strip_ns(p, sms[a], sns[b], cus);
                    if (q.M == 0 || q.N == 0) {
                        ts -= kLaunchFloorNs;
                        // no tiled block: the strips are the whole product
                        if (best.id < 0 || ts < best_t) {
                            best = {i, 1, sms[a], sns[b]};
                            best_t = ts;
                        }
                        continue;
                    }
                    const int e = edge_chunks(v, q) ? v.eff_unaligned_permille : eff;
                    int last = 0;
                    for (int want : kSplitCandidates) {
                        int splits, k_chunk;
                        split_k(q.K, want, splits, k_chunk);
                        if (splits <= last) continue;
                        last = splits;
                        if (split_workspace_bytes(q, splits) > workspace_bytes) break;
                        const long long grid =
                            ceil_div_ll(q.M, v.bm) * ceil_div_ll(q.N, v.bn) * splits * (long long)q.batch;
                        if (grid > INT_MAX) break;
                        const double t = estimate_ns(v, q, splits, k_chunk, cus, e) + ts;
                        if (best.id < 0 || t < best_t) {
                            best = {i, splits, sms[a], sns[b]};
                            best_t = t;
                        }
                    }
                }
            }
        }
    }
    return best;
}

}  // namespace sgemm
