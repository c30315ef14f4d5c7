// tropical_gemm_strided_batched: argument checks, kernel choice, launch.
//
// The batched tropical product with argmax of tropical-gemm PR #35
// ("feat: batched GPU ops with DLPack zero-copy output", Key changes).  That
// PR puts the batch on the third grid axis; here the batch and the output
// tiles share one flat grid so that the workgroup -> XCD remap in the kernel
// can keep neighbouring tiles of one batch entry on one XCD.  Which of
// A / B is row- or column-major is read from the strides (one kernel serves
// every layout; a column-major operand is transposed into LDS on load).
#include <cstdlib>
#include <cstring>
#include <string>

#include "internal.h"

namespace trop {

namespace {

bool env_flag(const char* name) {
    const char* v = std::getenv(name);
    return v && *v && std::strcmp(v, "0") != 0;
}

bool env_flag_off(const char* name) {
    const char* v = std::getenv(name);
    return v && std::strcmp(v, "0") == 0;
}

constexpr uint32_t kMaxGrid = 1u << 30;

uint32_t grid_for(int64_t work, int64_t per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g > kMaxGrid) g = kMaxGrid;
    return (uint32_t)g;
}

uint32_t zero_bits(trop_semiring sr, trop_dtype dt) {
    if (dt == TROP_I32) {
        const int32_t z = (sr == TROP_MAX_MUL) ? 0 : (sr == TROP_MIN_PLUS) ? (1 << 30) : -(1 << 30);
        uint32_t b;
        std::memcpy(&b, &z, 4);
        return b;
    }
    if (sr == TROP_MAX_PLUS) return 0xff800000u;  // -inf
    if (sr == TROP_MIN_PLUS) return 0x7f800000u;  // +inf
    return 0u;                                    // +0
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

trop_status check_gemm_args(trop_semiring sr, trop_dtype dt, trop_strides sA, trop_strides sB,
                            trop_strides sC, int64_t m, int64_t n, int64_t k, int64_t batch) {
    if (sr < TROP_MAX_PLUS || sr > TROP_MAX_MUL)
        return fail(TROP_ERR_INVALID_ARGUMENT, "unknown semiring " + std::to_string((int)sr));
    if (dt != TROP_F32 && dt != TROP_I32)
        return fail(TROP_ERR_INVALID_ARGUMENT, "unknown dtype " + std::to_string((int)dt));
    if (ring_index(sr, dt) < 0) return fail(TROP_ERR_UNSUPPORTED, "no such semiring / dtype pair");
    if (m < 0 || n < 0 || k < 0 || batch < 0)
        return fail(TROP_ERR_INVALID_ARGUMENT, "negative size");
    if (k > INT32_MAX) return fail(TROP_ERR_INVALID_ARGUMENT, "k must be < 2^31 (int32 argmax)");
    const trop_strides* all[3] = {&sA, &sB, &sC};
    for (const trop_strides* s : all)
        if (s->row < 0 || s->col < 0 || s->batch < 0)
            return fail(TROP_ERR_INVALID_ARGUMENT, "negative stride");
    return TROP_OK;
}

// Split-K policy: split only a product with fewer output tiles (times
// batch) than a 256-CU device has CUs, and only when every range keeps at
// least kSplitMinK terms (one resident K-block); aim at about kSplitTarget
// (tile, range) units.  A tiny product -- at most kSplitTinyUnits (tile,
// 256-term block) pairs, i.e. busy on a quarter of the CUs at most -- takes
// ranges of kSplitTinyK terms instead: a single 64 x 64 tile with K = 256
// runs its four slices one after another on one CU, and as four ranges on
// four CUs plus the merge it finished in about two thirds of the time.
// (128 and more pairs measured slower split that way.)
constexpr int64_t kSplitTarget = 512;
constexpr int64_t kSplitMinK = 256;
constexpr int64_t kSplitAlign = 256;  // ranges are whole resident K-blocks
constexpr int64_t kSplitTinyUnits = 64;
constexpr int64_t kSplitTinyK = 64;  // one slice of the split kernels
// Products of at most this many 64 x 64 tiles take 64 x 16 tiles (with 256
// tiles, a 64 x 16 grid of 1024 measured slower: 23 -> 35 us on 32 x 256 x
// 128 x 256; with 128, faster: 21.3 -> 18.5 us on 8 x 256^3)
constexpr int64_t kTiny16Tiles = 128;
// Products with K <= kSmallKMax, 192..256 columns and at least
// kSmallKMinRows rows (times batch) take the short-K kernel
// (TROPICAL_GEMM_SMALLK=0: never).  65536 x 256 x 16 with argmax: 49.6 ->
// 39.5 us (column-major A 54.8 -> 39.5), K = 4: 44 -> 27.5 us; with fewer
// rows its per-workgroup set-up shows (16384 x 256 x 16: 16.6 -> 19.0 us),
// with fewer columns its idle lanes (131072 x 128 x 16: 50.6 -> 67.8 us).
// 128..191 columns (two rows per lane group): from kSmallKMinRows128 rows
// (131072 x 128 x 16: 49.7 -> 41.5 us; 65536 x 128 x 16: 27.5 -> 26.4 us;
// fewer than 128 columns measured no faster).
constexpr int64_t kSmallKMax = 16;
constexpr int64_t kSmallKMinN = 128;
constexpr int64_t kSmallKMinRows = 32768;
constexpr int64_t kSmallKMinRows128 = 65536;
// Products with a longer K take the global-resolve argmax kernel
// (TROPICAL_GEMM_GRES_MIN_K overrides, for measurements).
const int64_t kGresMinK = [] {
    const char* v = std::getenv("TROPICAL_GEMM_GRES_MIN_K");
    return v && *v ? (int64_t)std::strtoll(v, nullptr, 10) : (int64_t)256;
}();

// Float mode of int32 max-plus / min-plus products: the domain pre-pass
// runs kFmSlots workgroups, one flag each, in the workspace; it is taken
// for products of at least kFmMinTerms terms (below that the pre-pass and
// the second, gated launch cost more than the float arithmetic saves).
// TROPICAL_GEMM_INT_FLOAT=0 never takes it, =1 takes it at any size.
constexpr int kFmSlots = 256;
constexpr size_t kFmBytes = kFmSlots * sizeof(int32_t);
constexpr int64_t kFmMinTerms = int64_t(1) << 32;

int fm_knob() {
    const char* v = std::getenv("TROPICAL_GEMM_INT_FLOAT");
    if (!v || !*v) return -1;
    return v[0] == '0' ? 0 : 1;
}

bool fm_size_ok(int64_t m, int64_t n, int64_t k, int64_t batch) {
    const int knob = fm_knob();
    if (knob >= 0) return knob == 1;
    int64_t t = 0;
    if (__builtin_mul_overflow(m, n, &t) || __builtin_mul_overflow(t, k, &t) || __builtin_mul_overflow(t, batch, &t))
        return true;
    return t >= kFmMinTerms;
}

// Transposed copies of the operands: an argmax product with a long K whose
// B is row-major (j unit-stride) copies B into the workspace as (batch, n,
// k), k unit-stride, and one whose A is column-major (i unit-stride) copies
// A as (batch, m, k), so that the global-resolve kernel reads both
// operands in 16-byte quads along k.  A copy moves 8 bytes per element,
// each of which the product then reads m / 64 (B) or n / 64 (A) times:
// taken for at least kBtMinRows rows, kBtMinTerms terms and K >= kBtMinK
// (4096^3 min-plus f32: 3.45 -> 2.88 ms; 2048^3 max-plus: 472 -> 388 us;
// 4096 x 300 x 4096: 306 -> 310 us, not taken).  The copies sit after the
// float-mode flags, B's first.  TROPICAL_GEMM_B_TRANSPOSE=0 never takes
// them, =1 at any size with K > kGresMinK.
constexpr size_t kBtOffset = 1024;
static_assert(kFmBytes <= kBtOffset, "the float-mode flags overlap the operand copies");
constexpr int64_t kBtMinRows = 256;
constexpr int64_t kBtMinTerms = int64_t(1) << 30;
constexpr int64_t kBtMinK = 512;

int bt_knob() {
    const char* v = std::getenv("TROPICAL_GEMM_B_TRANSPOSE");
    if (!v || !*v) return -1;
    return v[0] == '0' ? 0 : 1;
}

SplitK plan_splitk(int64_t m, int64_t n, int64_t k, int64_t batch) {
    SplitK s;
    // (K < 2^31, as the calls require: the sizes below then stay far from
    // overflow, units being at most kSplitTarget / 2)
    if (m <= 0 || n <= 0 || batch <= 0 || k <= 0 || k >= (int64_t(1) << 31)) return s;
    int64_t units = 0;
    if (__builtin_mul_overflow((m + 63) / 64, (n + 63) / 64, &units) ||
        __builtin_mul_overflow(units, batch, &units))
        return s;
    if (units > kSplitTarget / 2) return s;
    const int64_t blocks = k / 256 > 1 ? k / 256 : 1;
    const bool tiny = units * blocks <= kSplitTinyUnits && !env_flag_off("TROPICAL_SPLITK_TINY");
    const int64_t min_k = tiny ? kSplitTinyK : kSplitMinK;
    const int64_t align = tiny ? kSplitTinyK : kSplitAlign;
    if (k < 2 * min_k) return s;
    int64_t want = (kSplitTarget + units - 1) / units;
    if (want > k / min_k) want = k / min_k;
    if (want < 2) return s;
    int64_t chunk = (k + want - 1) / want;
    chunk = (chunk + align - 1) / align * align;
    const int64_t ks = (k + chunk - 1) / chunk;
    if (ks < 2) return s;
    s.ksplit = ks;
    s.kchunk = chunk;
    const size_t part = (size_t)(ks * batch * m * n) * 4;
    s.bytes = 2 * ((part + 255) / 256 * 256);
    return s;
}

bool kcol_b_pays(int64_t m, int64_t n, int64_t k, int64_t batch) {
    const int knob = bt_knob();
    if (knob == 0 || m <= 0 || n <= 0 || batch <= 0 || k <= kGresMinK || k % 4 != 0) return false;
    if (plan_splitk(m, n, k, batch).bytes > 0) return false;
    if (knob > 0) return true;
    int64_t t = 0;
    const bool many = __builtin_mul_overflow(m, n, &t) || __builtin_mul_overflow(t, k, &t) ||
                      __builtin_mul_overflow(t, batch, &t) || t >= kBtMinTerms;
    return m >= kBtMinRows && k >= kBtMinK && many;
}

// The operand copies run_gemm makes for these strides (none: not for this
// layout or shape).  A is copied when column-major, B when row-major, A is
// then read along k and the product has an argmax output; the pointers'
// 16-byte alignment is checked at the call.
OperandCopies plan_copies(trop_strides sA, trop_strides sB, bool argmax, int64_t m, int64_t n, int64_t k,
                          int64_t batch) {
    OperandCopies c;
    if (!kcol_b_pays(m, n, k, batch)) return c;
    const bool a_along_k = sA.col == 1 && sA.row % 4 == 0 && sA.batch % 4 == 0;
    const bool a_copy = sA.col != 1 && sA.row == 1;
    if (!a_along_k && !a_copy) return c;
    // (B only with an argmax output: the value-only kernel reads a
    // row-major B as fast)
    const bool b_copy = argmax && sB.col == 1;
    if (!a_copy && !b_copy) return c;
    int64_t ea = 0, eb = 0;
    if (__builtin_mul_overflow(batch, k, &ea) || __builtin_mul_overflow(ea, m, &ea) || ea > (INT64_MAX >> 4) ||
        __builtin_mul_overflow(batch, k, &eb) || __builtin_mul_overflow(eb, n, &eb) || eb > (INT64_MAX >> 4))
        return c;
    size_t off = kBtOffset;
    if (b_copy) {
        c.b = true;
        c.b_off = off;
        off += (size_t)((eb * 4 + 255) / 256 * 256);
    }
    if (a_copy) {
        c.a = true;
        c.a_off = off;
        off += (size_t)((ea * 4 + 255) / 256 * 256);
    }
    c.bytes = off;
    return c;
}

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t batch) {
    if (m <= 0 || n <= 0 || k <= 0 || batch <= 0) return 0;
    const SplitK sk = plan_splitk(m, n, k, batch);
    if (sk.bytes > 0) return sk.bytes;
    return fm_size_ok(m, n, k, batch) ? kFmBytes : 0;
}

trop_status run_gemm(int dev, trop_semiring sr, trop_dtype dt, const void* A, trop_strides sA,
                     const void* B, trop_strides sB, void* C, trop_strides sC, int32_t* argmax,
                     int64_t m, int64_t n, int64_t k, int64_t batch, hipStream_t stream, void* workspace,
                     size_t workspace_bytes, const GemmKRuns* kr) {
    if (m == 0 || n == 0 || batch == 0) return TROP_OK;
    const int ri = ring_index(sr, dt);
    if (k == 0) {
        TropFillParams f{};
        f.C = C;
        f.argmax = argmax;
        f.sc_row = sC.row;
        f.sc_col = sC.col;
        f.sc_batch = sC.batch;
        f.m = m;
        f.n = n;
        f.batch = batch;
        f.zero_bits = zero_bits(sr, dt);
        return launch(dev, K_FILL, TROP_K_FILL, grid_for(m * n * batch, 256), 256, &f, stream);
    }

    TropGemmParams p{};
    p.A = A;
    p.B = B;
    p.C = C;
    p.argmax = argmax;
    p.sa_row = sA.row;
    p.sa_col = sA.col;
    p.sa_batch = sA.batch;
    p.sb_row = sB.row;
    p.sb_col = sB.col;
    p.sb_batch = sB.batch;
    p.sc_row = sC.row;
    p.sc_col = sC.col;
    p.sc_batch = sC.batch;
    p.m = m;
    p.n = n;
    p.k = k;
    p.batch = batch;
    p.ksplit = 1;
    p.kchunk = k;
    p.c_split = 0;

    // two-level k (contracted axes on both sides of the free ones): read
    // along k, 16-byte vectors inside the runs
    const bool a_two = kr && kr->a_run > 0, b_two = kr && kr->b_run > 0;
    if (a_two) {
        p.a_krun = kr->a_run;
        p.sa_khi = kr->a_hi;
    }
    if (b_two) {
        p.b_krun = kr->b_run;
        p.sb_khi = kr->b_hi;
    }
    if (env_flag("TROPICAL_FORCE_SIMPLE_GEMM")) {
        return launch(dev, (KernelId)(K_GEMM_SIMPLE_MAXPLUS_F32 + ri), TROP_K_GEMM_SIMPLE,
                      grid_for(m * n * batch, 256), 256, &p, stream);
    }
    // A short K with 128..256 columns: B held in registers, rows of A
    // streamed (gemm_smallk_body; not under a forced GEMM setting, which
    // the tests use to drive the tiled kernels at these shapes)
    {
        const char* forced = std::getenv("TROPICAL_GEMM_SETTING");
        const bool c_ok = sC.col == 1 && sC.row % 4 == 0 && sC.batch % 4 == 0 && aligned16(C) &&
                          (!argmax || aligned16(argmax));
        if (k >= 1 && k <= kSmallKMax && n >= kSmallKMinN && n <= 256 && n % 4 == 0 &&
            m * batch >= (n >= 192 ? kSmallKMinRows : kSmallKMinRows128) &&
            c_ok && !(forced && *forced) && !env_flag_off("TROPICAL_GEMM_SMALLK")) {
            const KernelId id = (KernelId)(K_GEMM_SMALLK_MAXPLUS_F32 + ri);
            int per_cu = kernel_occupancy(dev, id);
            if (per_cu < 1) per_cu = 1;
            const int64_t units = (m + 31) / 32 * batch;  // units of 32 rows
            const int64_t slots = (int64_t)device_cu_count(dev) * per_cu;
            return launch(dev, id, TROP_K_GEMM_TILED, (uint32_t)(units < slots ? units : slots), 256, &p, stream);
        }
    }

    // A: row-major (k unit-stride), column-major (i unit-stride), or
    // neither (element-wise loads along k).
    if (a_two) {
        p.a_mode = TROP_LOAD_K_CONTIG;
        p.a_vec = aligned16(A) && sA.row % 4 == 0 && sA.batch % 4 == 0 && kr->a_hi % 4 == 0;
    } else if (sA.col == 1) {
        p.a_mode = TROP_LOAD_K_CONTIG;
        p.a_vec = aligned16(A) && sA.row % 4 == 0 && sA.batch % 4 == 0;
    } else if (sA.row == 1) {
        p.a_mode = TROP_LOAD_MN_CONTIG;
        p.a_vec = aligned16(A) && sA.col % 4 == 0 && sA.batch % 4 == 0;
    } else {
        p.a_mode = TROP_LOAD_K_CONTIG;
        p.a_vec = 0;
    }
    // B: row-major (j unit-stride), column-major (k unit-stride), or neither.
    if (b_two) {
        p.b_mode = TROP_LOAD_K_CONTIG;
        p.b_vec = aligned16(B) && sB.col % 4 == 0 && sB.batch % 4 == 0 && kr->b_hi % 4 == 0;
    } else if (sB.col == 1) {
        p.b_mode = TROP_LOAD_MN_CONTIG;
        p.b_vec = aligned16(B) && sB.row % 4 == 0 && sB.batch % 4 == 0;
    } else if (sB.row == 1) {
        p.b_mode = TROP_LOAD_K_CONTIG;
        p.b_vec = aligned16(B) && sB.col % 4 == 0 && sB.batch % 4 == 0;
    } else {
        p.b_mode = TROP_LOAD_K_CONTIG;
        p.b_vec = 0;
    }
    // transposed copies of the operands in the workspace (see kBtOffset):
    // both are then read along k in 16-byte quads, by the global-resolve
    // kernel (not under a forced wide or narrow setting)
    const char* setting = std::getenv("TROPICAL_GEMM_SETTING");
    const bool setting_local = setting && (std::strcmp(setting, "wide") == 0 || std::strcmp(setting, "narrow") == 0);
    const OperandCopies cp = workspace && !a_two && !b_two && !setting_local
                                 ? plan_copies(sA, sB, argmax != nullptr, m, n, k, batch)
                                 : OperandCopies();
    if (cp.bytes > 0 && workspace_bytes >= cp.bytes && aligned16(workspace)) {
        // one operand's copy: output (batch, rows, k) contiguous, read
        // through the operand's strides
        auto copy = [&](const void* src, int64_t rows, int64_t s_batch, int64_t s_rows, int64_t s_k,
                        size_t off) -> trop_status {
            const int64_t oshape[3] = {batch, rows, k}, ostride[3] = {s_batch, s_rows, s_k};
            GatherPlan g{};
            trop_status st = plan_gather(3, oshape, ostride, 0, nullptr, nullptr, &g);
            if (st != TROP_OK) return st;
            const void* gin[1] = {src};
            void* gout[1] = {static_cast<char*>(workspace) + off};
            return run_gather(dev, g, 1, gin, gout, sr, dt, stream);
        };
        if (cp.a) {
            trop_status st = copy(A, m, sA.batch, sA.row, sA.col, cp.a_off);
            if (st != TROP_OK) return st;
            p.A = static_cast<char*>(workspace) + cp.a_off;
            p.sa_row = k;
            p.sa_col = 1;
            p.sa_batch = m * k;
            p.a_mode = TROP_LOAD_K_CONTIG;
            p.a_vec = 1;  // (k % 4 == 0, the copy 256-byte aligned)
        }
        // (B only when A is now read along k: its alignment is known here)
        if (cp.b && p.a_mode == TROP_LOAD_K_CONTIG && p.a_vec) {
            trop_status st = copy(B, n, sB.batch, sB.col, sB.row, cp.b_off);
            if (st != TROP_OK) return st;
            p.B = static_cast<char*>(workspace) + cp.b_off;
            p.sb_row = 1;
            p.sb_col = k;
            p.sb_batch = k * n;
            p.b_mode = TROP_LOAD_K_CONTIG;
            p.b_vec = 1;
        }
    }
    const int64_t tm = (m + 63) / 64, tn = (n + 63) / 64;
    if (tm > INT32_MAX || tn > INT32_MAX) return fail(TROP_ERR_INVALID_ARGUMENT, "matrix too large");
    p.tiles_m = (int32_t)tm;
    p.tiles_n = (int32_t)tn;
    p.swizzle = env_flag("TROPICAL_NO_XCD_SWIZZLE") ? 0 : 1;
    p.group_rows = TROP_GEMM_GROUP_ROWS;
    if (const char* g = std::getenv("TROPICAL_GEMM_GROUP_ROWS")) {  // tuning knob: tile-rows per group
        const long v = std::strtol(g, nullptr, 10);
        if (v >= 1 && v <= 64) p.group_rows = (int32_t)v;
    }
    if (env_flag("TROPICAL_GEMM_ROW_RASTER")) p.group_rows = 1;
    // split K into ranges when the workspace allows and the shape asks for it:
    // partials go to [split][batch][m][n] in the workspace
    const SplitK sk = workspace ? plan_splitk(m, n, k, batch) : SplitK();
    const bool split = sk.ksplit > 1 && workspace_bytes >= sk.bytes && !env_flag("TROPICAL_NO_SPLIT_K");
    const int64_t part_elems = split ? sk.ksplit * batch * m * n : 0;
    if (split) {
        p.ksplit = sk.ksplit;
        p.kchunk = sk.kchunk;
        p.c_split = batch * m * n;
        p.C = workspace;
        p.argmax = argmax ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + sk.bytes / 2) : nullptr;
        p.sc_row = n;
        p.sc_col = 1;
        p.sc_batch = m * n;
        (void)part_elems;
    }
    int64_t total = tm * tn * batch * p.ksplit;
    // 32-bit tile decode with magic-number division (no 64-bit divides per tile)
    if (total < (int64_t(1) << 31) && !env_flag("TROPICAL_GEMM_COORD64")) {
        p.coord32 = 1;
        if (tm * tn >= 2) magic_u31((uint64_t)(tm * tn), &p.tl_m, &p.tl_s);
        if (tn >= 2) magic_u31((uint64_t)tn, &p.tn_m, &p.tn_s);
        if (p.ksplit >= 2) magic_u31((uint64_t)p.ksplit, &p.ks_m, &p.ks_s);
        magic_u31((uint64_t)(p.group_rows * tn), &p.gr_m, &p.gr_s);
    }
    // without an argmax output the value-only kernel skips the chunk record
    // and the re-scan
    // With an argmax, products of fewer than two tiles per CU take the
    // narrow setting (one workgroup per CU, loads ahead, K-block 256): the
    // wide one's second workgroup would have no tile.
    bool narrow = argmax && total < 2 * (int64_t)device_cu_count(dev);
    // A long K resolves each output's argmax once per tile from global
    // memory instead of once per resident K-block from LDS, where both
    // operands are read along k in 16-byte quads (K a multiple of 4); the
    // other layouts would re-read a strided operand element by element.
    const bool kvec = p.a_mode == TROP_LOAD_K_CONTIG && p.a_vec && p.b_mode == TROP_LOAD_K_CONTIG && p.b_vec &&
                      k % 4 == 0;
    bool gres = argmax && k > kGresMinK && kvec;
    if (const char* f = std::getenv("TROPICAL_GEMM_SETTING")) {  // tests: "wide", "narrow" or "global"
        if (std::strcmp(f, "wide") == 0) narrow = gres = false;
        if (std::strcmp(f, "narrow") == 0) {
            narrow = argmax;
            gres = false;
        }
        if (std::strcmp(f, "global") == 0) gres = argmax;
    }
    // One 16-column group per thread, in tiles of 64 rows x 16 columns:
    // products with at most 16 columns (a 64-column tile would be three
    // quarters padding), and small products (at most kTiny16Tiles 64 x 64
    // tiles), which then spread over four times the workgroups.  The wide
    // forms only: not with split K, the global resolve or a forced narrow
    // setting.  TROPICAL_GEMM_NO_NARROW_N=1: the 64-column forms.
    // Float mode of an int32 product (its kernels have 64-column tiles); the
    // domain pre-pass reads plain strides: not with a two-level k.
    const bool fm = dt == TROP_I32 && sr != TROP_MAX_MUL && !split && workspace && workspace_bytes >= kFmBytes &&
                    !a_two && !b_two && fm_size_ok(m, n, k, batch);
    const bool forced_narrow = setting && std::strcmp(setting, "narrow") == 0;
    const bool n16 = !split && !gres && !fm && !forced_narrow && !env_flag("TROPICAL_GEMM_NO_NARROW_N") &&
                     (n <= 16 || (tm * tn * batch <= kTiny16Tiles && !env_flag_off("TROPICAL_GEMM_TINY16")));
    if (n16) {
        narrow = false;
        const int64_t tn16 = (n + 15) / 16;
        p.tiles_n = (int32_t)tn16;
        total = tm * tn16 * batch * p.ksplit;
        if (p.coord32) {
            if (tm * tn16 >= 2) magic_u31((uint64_t)(tm * tn16), &p.tl_m, &p.tl_s);
            if (tn16 >= 2) magic_u31((uint64_t)tn16, &p.tn_m, &p.tn_s);
            magic_u31((uint64_t)(p.group_rows * tn16), &p.gr_m, &p.gr_s);
        }
    }
    // the global-resolve instance with both operands' loads fixed at
    // compile time (16-byte vectors along k) where the layout is that one
    // (TROPICAL_GEMM_FIXED_LAYOUT=0: always the general instance)
    // Instances with both operands' loads fixed at compile time (16-byte
    // vectors; fewer registers) where the layout is theirs: the global
    // resolve with A and B read along k, the wide form with A along k and B
    // along its rows (row-major A and B).  TROPICAL_GEMM_FIXED_LAYOUT=0:
    // always the general instances.
    const bool fixed_ok = !env_flag_off("TROPICAL_GEMM_FIXED_LAYOUT");
    const bool kmvec = p.a_mode == TROP_LOAD_K_CONTIG && p.a_vec && p.b_mode == TROP_LOAD_MN_CONTIG && p.b_vec;
    // (the fixed global-resolve instance addresses a tile's panels with
    // 32-bit byte offsets: every element within 2^29 of the panel's start)
    const int64_t pan_lim = int64_t(1) << 29;
    const int64_t a_kspan = a_two ? (k - 1) / p.a_krun * p.sa_khi + p.a_krun : k;
    const int64_t b_kspan = b_two ? (k - 1) / p.b_krun * p.sb_khi + p.b_krun : k;
    const bool pan32 = 63 * p.sa_row + a_kspan < pan_lim && 63 * p.sb_col + b_kspan < pan_lim;
    // (the fixed instances are built without the two-level k; the km form
    // has a second instance with it)
    const bool fixed = gres && kvec && fixed_ok && pan32 && !a_two && !b_two;
    const bool fixed_km = !gres && !narrow && kmvec && fixed_ok;
    // (the 16-column forms have the two-level k)
    const KernelId km_id = n16 ? K_GEMM_TILED_KM1_MAXPLUS_F32
                               : (a_two || b_two ? K_GEMM_TILED_KMR_MAXPLUS_F32 : K_GEMM_TILED_KM_MAXPLUS_F32);
    const KernelId wide_id = n16 ? K_GEMM_TILED_W1_MAXPLUS_F32 : K_GEMM_TILED_MAXPLUS_F32;
    const KernelId vo_id = n16 ? K_GEMM_TILED_VO1_MAXPLUS_F32
                               : (a_two || b_two ? K_GEMM_TILED_VOR_MAXPLUS_F32 : K_GEMM_TILED_VO_MAXPLUS_F32);
    const KernelId kid =
        split ? (KernelId)((argmax ? K_GEMM_TILED_SPLIT_MAXPLUS_F32 : K_GEMM_TILED_VO_SPLIT_MAXPLUS_F32) + ri)
              : (KernelId)((argmax ? (gres     ? (fixed ? K_GEMM_TILED_GKK_MAXPLUS_F32 : K_GEMM_TILED_G_MAXPLUS_F32)
                                      : narrow ? K_GEMM_TILED_N_MAXPLUS_F32
                                               : (fixed_km ? km_id : wide_id))
                                   : vo_id) +
                         ri);
    // Persistent grid: as many workgroups as the CUs hold at once (LDS and
    // registers decide), each walking a stream of tiles.  A multiple of 8
    // keeps every workgroup's tiles on one XCD.
    auto launch_tiled = [&](KernelId id) -> trop_status {
        int per_cu = kernel_occupancy(dev, id);
        if (per_cu < 1) per_cu = 1;
        int64_t slots = (int64_t)device_cu_count(dev) * per_cu / 8 * 8;
        if (slots < 8) slots = 8;
        if (const char* cap = std::getenv("TROPICAL_GEMM_MAX_WORKGROUPS")) {  // tuning knob
            long v = std::strtol(cap, nullptr, 10);
            if (v >= 8) slots = v / 8 * 8;
        }
        const uint32_t grid = (uint32_t)(total < slots ? total : slots);
        const int block = kernel_block(dev, id);  // the launch bound the kernel was built with
        if (block != 256 && block != 512 && block != 1024)
            return fail(TROP_ERR_HIP, std::string(kernel_name(id)) + ": unexpected launch bound " +
                                          std::to_string(block));
        return launch(dev, id, TROP_K_GEMM_TILED, grid, (uint32_t)block, &p, stream);
    };
    // Float mode of an int32 max-plus / min-plus product: the domain
    // pre-pass writes its flags into the workspace, then the float-mode
    // kernel and the int32 kernel are both enqueued, each gated on the flags
    // so that exactly one of them computes.  No host round trip.
    if (fm) {
        TropDomainParams d{};
        d.A = static_cast<const int32_t*>(A);
        d.B = static_cast<const int32_t*>(B);
        d.flags = static_cast<int32_t*>(workspace);
        d.sa_row = sA.row;
        d.sa_col = sA.col;
        d.sa_batch = sA.batch;
        d.sb_row = sB.row;
        d.sb_col = sB.col;
        d.sb_batch = sB.batch;
        d.m = m;
        d.n = n;
        d.k = k;
        d.batch = batch;
        const int mp = sr == TROP_MIN_PLUS ? 1 : 0;
        trop_status st = launch(dev, (KernelId)(K_GEMM_DOMAIN_MAXPLUS + mp), TROP_K_GEMM_DOMAIN, kFmSlots, 256, &d,
                                stream);
        if (st != TROP_OK) return st;
        p.mode_flags = d.flags;
        p.mode_slots = kFmSlots;
        p.mode_run = 1;
        const KernelId fid = (KernelId)((argmax ? (gres     ? K_GEMM_FMG_MAXPLUS
                                                   : narrow ? K_GEMM_FMN_MAXPLUS
                                                            : (fixed_km ? K_GEMM_FMKM_MAXPLUS : K_GEMM_FM_MAXPLUS))
                                                : K_GEMM_FMVO_MAXPLUS) + mp);
        st = launch_tiled(fid);
        if (st != TROP_OK) return st;
        p.mode_run = 0;
        return launch_tiled(kid);
    }
    trop_status st = launch_tiled(kid);
    if (st != TROP_OK || !split) return st;
    TropSplitMergeParams mp{};
    mp.pval = p.C;
    mp.pidx = p.argmax;
    mp.C = C;
    mp.argmax = argmax;
    mp.sc_row = sC.row;
    mp.sc_col = sC.col;
    mp.sc_batch = sC.batch;
    mp.m = m;
    mp.n = n;
    mp.batch = batch;
    mp.ksplit = sk.ksplit;
    // about one lane per 8 ranges (each lane keeps 8 loads in flight)
    mp.lanes = 1;
    while (mp.lanes < TROP_MERGE_LANES && mp.lanes * 8 < sk.ksplit) mp.lanes *= 2;
    return launch(dev, (KernelId)(K_GEMM_SPLITK_MERGE_MAXPLUS_F32 + ri), TROP_K_GEMM_SPLITK_MERGE,
                  grid_for(m * n * batch * mp.lanes, 256), 256, &mp, stream);
}

}  // namespace trop

namespace {

trop_status gemm_entry(trop_semiring semiring, trop_dtype dtype, const void* A, trop_strides sA, const void* B,
                       trop_strides sB, void* C, trop_strides sC, int32_t* argmax, int64_t m, int64_t n,
                       int64_t k, int64_t batch, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace trop;
    trop_status st = check_gemm_args(semiring, dtype, sA, sB, sC, m, n, k, batch);
    if (st != TROP_OK) return st;
    if (m == 0 || n == 0 || batch == 0) return ok();
    const SplitK sk = plan_splitk(m, n, k, batch);
    if (workspace && sk.bytes > 0 && workspace_bytes < sk.bytes)
        return fail(TROP_ERR_WORKSPACE_TOO_SMALL,
                    "workspace needs " + std::to_string(sk.bytes) + " bytes, got " + std::to_string(workspace_bytes));
    // (the float mode of int32 products and the transposed operand copies use a
    // workspace when one of their size is given, and are skipped otherwise)
    const size_t ws_base = gemm_workspace_bytes(m, n, k, batch);
    const size_t ws_bt = workspace ? plan_copies(sA, sB, argmax != nullptr, m, n, k, batch).bytes : 0;
    const size_t ws_need = ws_bt > ws_base && workspace_bytes >= ws_bt ? ws_bt : ws_base;
    int dev = -1;
    st = current_device(&dev);
    if (st != TROP_OK) return st;

    int64_t spanA = 0, spanB = 0, spanC = 0;
    if (k > 0) {
        const int64_t eA[3] = {batch, m, k}, sa[3] = {sA.batch, sA.row, sA.col};
        const int64_t eB[3] = {batch, k, n}, sb[3] = {sB.batch, sB.row, sB.col};
        if (!max_offset(3, eA, sa, &spanA) || !max_offset(3, eB, sb, &spanB))
            return fail(TROP_ERR_INVALID_ARGUMENT, "operand extent overflows");
        ++spanA;
        ++spanB;
        st = check_device_span(A, dev, spanA, 4, "A");
        if (st != TROP_OK) return st;
        st = check_device_span(B, dev, spanB, 4, "B");
        if (st != TROP_OK) return st;
    }
    const int64_t eC[3] = {batch, m, n}, sc[3] = {sC.batch, sC.row, sC.col};
    if (!max_offset(3, eC, sc, &spanC)) return fail(TROP_ERR_INVALID_ARGUMENT, "C extent overflows");
    ++spanC;
    st = check_device_span(C, dev, spanC, 4, "C");
    if (st != TROP_OK) return st;
    if (argmax) {
        st = check_device_span(argmax, dev, spanC, 4, "argmax");
        if (st != TROP_OK) return st;
    }
    const bool use_ws = workspace && ws_need > 0 && workspace_bytes >= ws_need;
    if (use_ws) {
        st = check_device_span(workspace, dev, (int64_t)(ws_need / 4), 4, "workspace");
        if (st != TROP_OK) return st;
    }
    st = run_gemm(dev, semiring, dtype, A, sA, B, sB, C, sC, argmax, m, n, k, batch,
                  static_cast<hipStream_t>(stream), use_ws ? workspace : nullptr, use_ws ? ws_need : 0);
    return st == TROP_OK ? ok() : st;
}

}  // namespace

extern "C" trop_status tropical_gemm_strided_batched(trop_semiring semiring, trop_dtype dtype,
                                                     const void* A, trop_strides sA, const void* B,
                                                     trop_strides sB, void* C, trop_strides sC,
                                                     int32_t* argmax, int64_t m, int64_t n, int64_t k,
                                                     int64_t batch, void* stream) {
    return gemm_entry(semiring, dtype, A, sA, B, sB, C, sC, argmax, m, n, k, batch, nullptr, 0, stream);
}

extern "C" trop_status tropical_gemm_strided_batched_ws(trop_semiring semiring, trop_dtype dtype,
                                                        const void* A, trop_strides sA, const void* B,
                                                        trop_strides sB, void* C, trop_strides sC,
                                                        int32_t* argmax, int64_t m, int64_t n, int64_t k,
                                                        int64_t batch, void* workspace, size_t workspace_bytes,
                                                        void* stream) {
    return gemm_entry(semiring, dtype, A, sA, B, sB, C, sC, argmax, m, n, k, batch, workspace, workspace_bytes,
                      stream);
}

extern "C" trop_status tropical_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int64_t batch,
                                                    size_t* bytes) {
    using namespace trop;
    if (!bytes) return fail(TROP_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (m < 0 || n < 0 || k < 0 || batch < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative size");
    *bytes = gemm_workspace_bytes(m, n, k, batch);
    return ok();
}

extern "C" trop_status tropical_gemm_workspace_size_strided(trop_strides sA, trop_strides sB, int with_argmax,
                                                            int64_t m, int64_t n, int64_t k, int64_t batch,
                                                            size_t* bytes) {
    using namespace trop;
    if (!bytes) return fail(TROP_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (m < 0 || n < 0 || k < 0 || batch < 0) return fail(TROP_ERR_INVALID_ARGUMENT, "negative size");
    if (sA.row < 0 || sA.col < 0 || sA.batch < 0 || sB.row < 0 || sB.col < 0 || sB.batch < 0)
        return fail(TROP_ERR_INVALID_ARGUMENT, "negative stride");
    const size_t base = gemm_workspace_bytes(m, n, k, batch);
    const size_t bt = plan_copies(sA, sB, with_argmax != 0, m, n, k, batch).bytes;
    *bytes = bt > base ? bt : base;
    return ok();
}
