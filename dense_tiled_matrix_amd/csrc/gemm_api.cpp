// gemm_api.cpp -- the C ABI declared in dtm_gemm.h: argument checks, the
// tile-config selector, and kernel dispatch on the caller's stream.
//
// The host side of "Chapter 13: The Blocked Matmul Kernel" section 13.1's
// wrapper: check the shapes, size the launch grid as
// (cdiv(M, BLOCK_M), cdiv(N, BLOCK_N)) with cdiv(K, BLOCK_K) K-iterations per
// tile, and pass the six element strides through.  Unlike the pages' wrapper
// the output is caller-owned and every check runs before anything is
// launched ("Triton matmul" notes: a failure before the GPU is reached is the
// one to want).
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <optional>

#include "dtm_gemm.h"
#include "host_util.h"
#include "launch.h"

namespace dtm {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool env_pointer_checks()
{
    const char *v = std::getenv("DTM_CHECK_POINTERS");
    return v && *v && std::strcmp(v, "0") != 0;
}
std::atomic<bool> g_pointer_checks{env_pointer_checks()};

// DTM_GEMM_FORCE: a tile configuration for the calls that pass none (gemm(),
// and gemm_plan() / gemm_ex() / gemm_ex_noalloc() with force == NULL), so a
// sweep can drive an unmodified caller.  Read once, when the library is
// loaded; unset or empty means off.  Comma-separated fields, each either
// "BMxBNxBK" (the tile) or key=value with key kernel (a dtm_kernel number or
// its gemm_kernel_name), split, threads or dp_rows.  A value that does not
// parse makes every such call return DTM_ERR_CONFIG.
struct EnvForce {
    bool on = false;
    bool bad = false;
    dtm_tile_config cfg{};
};

bool parse_i32(const char *s, const char *e, int32_t *out)
{
    if (s == e || e - s > 9)
        return false;
    int32_t v = 0;
    for (const char *q = s; q < e; ++q) {
        if (*q < '0' || *q > '9')
            return false;
        v = 10 * v + (*q - '0');
    }
    *out = v;
    return true;
}

bool parse_kernel(const char *s, const char *e, int32_t *out)
{
    if (parse_i32(s, e, out))
        return *out >= 0 && *out <= DTM_KERNEL_MFMA_F16_WAVEK;
    for (int32_t k = 0; k <= DTM_KERNEL_MFMA_F16_WAVEK; ++k) {
        const char *n = gemm_kernel_name(k);
        if (std::strlen(n) == static_cast<size_t>(e - s) && std::strncmp(n, s, e - s) == 0) {
            *out = k;
            return true;
        }
    }
    return false;
}

bool parse_field(const char *s, const char *e, dtm_tile_config *c)
{
    const char *eq = static_cast<const char *>(std::memchr(s, '=', e - s));
    if (!eq) {  // BMxBNxBK
        const char *x1 = static_cast<const char *>(std::memchr(s, 'x', e - s));
        const char *x2 = x1 ? static_cast<const char *>(std::memchr(x1 + 1, 'x', e - x1 - 1))
                            : nullptr;
        return x2 && parse_i32(s, x1, &c->block_m) && parse_i32(x1 + 1, x2, &c->block_n) &&
               parse_i32(x2 + 1, e, &c->block_k);
    }
    const size_t klen = eq - s;
    auto key = [&](const char *k) { return std::strlen(k) == klen && !std::strncmp(k, s, klen); };
    if (key("kernel"))
        return parse_kernel(eq + 1, e, &c->kernel);
    if (key("split"))
        return parse_i32(eq + 1, e, &c->split_k);
    if (key("threads"))
        return parse_i32(eq + 1, e, &c->threads);
    if (key("dp_rows"))
        return parse_i32(eq + 1, e, &c->dp_rows);
    return false;
}

EnvForce parse_env_force(const char *v)
{
    EnvForce f;
    if (!v || !*v)
        return f;
    f.on = true;
    const char *s = v;
    while (true) {
        const char *e = std::strchr(s, ',');
        if (!e)
            e = s + std::strlen(s);
        if (!parse_field(s, e, &f.cfg)) {
            f.bad = true;
            return f;
        }
        if (!*e)
            break;
        s = e + 1;
    }
    return f;
}

const EnvForce g_env_force = parse_env_force(std::getenv("DTM_GEMM_FORCE"));

// The configuration a call runs with: its own, else the environment's.
// Returns false when the environment's does not parse.
bool resolve_force(const dtm_tile_config *&force)
{
    if (force || !g_env_force.on)
        return true;
    if (g_env_force.bad)
        return false;
    force = &g_env_force.cfg;
    return true;
}

}  // namespace

bool pointer_checks_on() { return g_pointer_checks.load(std::memory_order_relaxed); }

int check_view_memory(uintptr_t lo, uintptr_t hi)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return DTM_ERR_POINTER;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, reinterpret_cast<const void *>(lo)) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error the query may leave
        return DTM_ERR_POINTER;
    }
    if (attr.type != hipMemoryTypeDevice || attr.device != dev)
        return DTM_ERR_POINTER;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, reinterpret_cast<hipDeviceptr_t>(lo)) != hipSuccess) {
        (void)hipGetLastError();
        return DTM_ERR_POINTER;
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base);
    return lo >= b && hi >= lo && hi - b <= size ? DTM_OK : DTM_ERR_POINTER;
}

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return DTM_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int known = g_device_ok[dev].load(std::memory_order_acquire);
        if (known == 1)
            return DTM_OK;
        if (known == 2)
            return DTM_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return DTM_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices)
        g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_release);
    return ok ? DTM_OK : DTM_ERR_DEVICE;
}

}  // namespace dtm

namespace {

using dtm::c_strides_ok;
using dtm::cdiv;
using dtm::check_device;
using dtm::GemmArgs;
using dtm::item_size;
using dtm::valid_dtype;
using dtm::view_range;

struct Call {
    int64_t M, N, K;
    const void *A;
    int64_t sam, sak;
    const void *B;
    int64_t sbk, sbn;
    const void *C;
    int64_t scm, scn;
    int in, out;
};

int validate(const Call &c)
{
    constexpr int64_t kMaxDim = 0x7fffffffLL;
    if (c.M < 0 || c.N < 0 || c.K < 0 || c.M > kMaxDim || c.N > kMaxDim || c.K > kMaxDim)
        return DTM_ERR_INVALID_DIM;
    if (!valid_dtype(c.in) || !valid_dtype(c.out))
        return DTM_ERR_DTYPE;
    if (c.M == 0 || c.N == 0)
        return DTM_OK;
    if (!c.C)
        return DTM_ERR_NULL_POINTER;
    if (c.K > 0 && (!c.A || !c.B))
        return DTM_ERR_NULL_POINTER;
    if (!c_strides_ok(c.M, c.N, c.scm, c.scn))
        return DTM_ERR_STRIDE;
    uintptr_t clo, chi;
    if (!view_range(c.C, c.M, c.N, c.scm, c.scn, item_size(c.out), clo, chi))
        return DTM_ERR_STRIDE;
    if (c.K > 0) {
        uintptr_t alo, ahi, blo, bhi;
        if (!view_range(c.A, c.M, c.K, c.sam, c.sak, item_size(c.in), alo, ahi) ||
            !view_range(c.B, c.K, c.N, c.sbk, c.sbn, item_size(c.in), blo, bhi))
            return DTM_ERR_STRIDE;
        if ((clo < ahi && alo < chi) || (clo < bhi && blo < chi))
            return DTM_ERR_ALIAS;
    }
    return DTM_OK;
}

// The MFMA kernels read 16-byte chunks along the unit-stride axis of each
// operand: A K- or M-contiguous, B N- or K-contiguous, every chunk start
// 16-byte aligned (the base and the leading dimension in bytes).  The same
// rule a tensor descriptor imposes ("Triton matmul", "Things that break"),
// used here to pick a kernel rather than to reject the call.  Returns the
// dtm_layout bits, or -1 when no aligned MFMA layout fits (fp16/bf16 views on
// 4-byte boundaries: mfma16_unaligned_layout; fp32: mfma32_layout).
int mfma_layout(const Call &c)
{
    if ((reinterpret_cast<uintptr_t>(c.A) & 15) || (reinterpret_cast<uintptr_t>(c.B) & 15))
        return -1;
    const int64_t per16 = 16 / item_size(c.in);
    int layout = 0;
    if (c.sak == 1 && c.sam % per16 == 0)
        ;
    else if (c.sam == 1 && c.sak % per16 == 0)
        layout |= DTM_LAYOUT_A_M_CONTIG;
    else
        return -1;
    if (c.sbn == 1 && c.sbk % per16 == 0)
        ;
    else if (c.sbk == 1 && c.sbn % per16 == 0)
        layout |= DTM_LAYOUT_B_K_CONTIG;
    else
        return -1;
    return layout;
}
bool is16(const Call &c) { return c.in == DTM_F16 || c.in == DTM_BF16; }

// fp16/bf16 views that mfma_layout() turns away but whose chunks still start
// on 4-byte boundaries (bases 4-byte aligned, the non-unit stride of each
// operand even): the register-staged kernel's range-checked form reads them
// with 16-byte copies at 4-byte alignment.  Returns the layout bits, or -1.
int mfma16_unaligned_layout(const Call &c)
{
    if (!is16(c) || (reinterpret_cast<uintptr_t>(c.A) & 3) ||
        (reinterpret_cast<uintptr_t>(c.B) & 3))
        return -1;
    int layout = 0;
    if (c.sak == 1 && c.sam % 2 == 0)
        ;
    else if (c.sam == 1 && c.sak % 2 == 0)
        layout |= DTM_LAYOUT_A_M_CONTIG;
    else
        return -1;
    if (c.sbn == 1 && c.sbk % 2 == 0)
        ;
    else if (c.sbk == 1 && c.sbn % 2 == 0)
        layout |= DTM_LAYOUT_B_K_CONTIG;
    else
        return -1;
    return layout;
}

// The fp32 matrix-core kernel also reads each operand along its unit-stride
// axis, but its range-checked form takes views off 16-byte boundaries too
// (element loads), so any fp32 view with a unit stride along one axis of
// each operand runs there.  *aligned: mfma_layout's 16-byte rule holds as
// well (the vector-load forms).  Returns the dtm_layout bits, or -1.
int mfma32_layout(const Call &c, bool *aligned)
{
    int layout = 0;
    if (c.sak == 1)
        ;
    else if (c.sam == 1)
        layout |= DTM_LAYOUT_A_M_CONTIG;
    else
        return -1;
    if (c.sbn == 1)
        ;
    else if (c.sbk == 1)
        layout |= DTM_LAYOUT_B_K_CONTIG;
    else
        return -1;
    if (aligned)
        *aligned = mfma_layout(c) == layout;
    return layout;
}

// Whether the wave-K kernel (128 x 128 tiles, the K loop split across the
// workgroup's waves) runs the call with `splits` K slices.
bool wavek_fits(const Call &c, int layout, int64_t splits)
{
    if (!is16(c) || layout < 0)
        return false;
    const GemmArgs a{c.M, c.N, c.K, c.A, c.sam, c.sak, c.B, c.sbk, c.sbn,
                     const_cast<void *>(c.C), c.scm, c.scn};
    return dtm::mfma16_wavek_fits(a, layout, splits);
}

// Byte extent of a view with non-negative strides (one past its last
// element, from its origin); UINT64_MAX when a stride is negative or the
// extent overflows.
uint64_t view_bytes(int64_t rows, int64_t cols, int64_t sr, int64_t sc, int64_t item)
{
    if (sr < 0 || sc < 0 || rows <= 0 || cols <= 0)
        return UINT64_MAX;
    const unsigned __int128 last = (unsigned __int128)(rows - 1) * (uint64_t)sr +
                                   (unsigned __int128)(cols - 1) * (uint64_t)sc + 1;
    const unsigned __int128 bytes = last * (uint64_t)item;
    return bytes > UINT64_MAX ? UINT64_MAX : (uint64_t)bytes;
}
uint64_t a_view_bytes(const Call &c) { return view_bytes(c.M, c.K, c.sam, c.sak, item_size(c.in)); }
uint64_t b_view_bytes(const Call &c) { return view_bytes(c.K, c.N, c.sbk, c.sbn, item_size(c.in)); }

void fill_grid(const Call &c, dtm_plan &p)
{
    p.grid_m = cdiv(c.M, p.block_m);
    p.grid_n = cdiv(c.N, p.block_n);
    const int64_t k_slice = cdiv(c.K, p.split_k > 0 ? p.split_k : 1);
    p.k_iters = cdiv(k_slice, p.block_k);
    p.ragged = (c.M % p.block_m) || (c.N % p.block_n) || (c.K % p.block_k) ? 1 : 0;
}

// Generic tile for a problem: the largest tile that still gives the chip a
// few hundred workgroups, down to 16 x 16.
void pick_generic(const Call &c, dtm_plan &p)
{
    struct T {
        int bm, bn, bk;
    };
    static const T order[] = {{64, 64, 16}, {32, 32, 16}, {16, 16, 16}};
    const T *pick = &order[2];
    for (const T &t : order) {
        if (cdiv(c.M, t.bm) * cdiv(c.N, t.bn) >= 512) {
            pick = &t;
            break;
        }
    }
    p.block_m = pick->bm;
    p.block_n = pick->bn;
    p.block_k = pick->bk;
}

// Whether the tile x tile x 32 pipelined kernel (tile 256 or 128) can run a
// problem with K in `splits` slices: its interior form (M, N multiples of
// the tile, K of 32 * splits) or its range-checked form.
bool dma_interior(const Call &c, int layout, int64_t splits, int tile = 256)
{
    return is16(c) && layout >= 0 && dtm::mfma16_dma_fits(c.M, c.N, c.K, splits, tile);
}
bool dma_ranged(const Call &c, int layout, int64_t splits, int tile = 256)
{
    return is16(c) && layout >= 0 &&
           dtm::mfma16_dma_ragged_fits(c.M, c.N, c.K, layout, a_view_bytes(c), b_view_bytes(c),
                                       splits, tile);
}
bool dma_any(const Call &c, int layout, int64_t splits, int tile = 256)
{
    return dma_interior(c, layout, splits, tile) || dma_ranged(c, layout, splits, tile);
}
bool is_dma_tile(int bm, int bn, int bk)
{
    return bm == bn && (bm == 256 || bm == 192 || bm == 128) && bk == 32;
}

// Tile of the pipelined kernel: 256 x 256 while there are more than
// SMALL_TILE_MAX such tiles, else 128 x 128 (four times the workgroups).
// Measured side by side (bf16 unless noted, TFLOP/s, 256 -> 128): 2048^3
// 419 -> 675 (256 was split 4 ways), 2560^3 668 -> 749, 1024x4096x4096
// 644 -> 801, 8192x1024x8192 (128 tiles of 256) 897 -> 967; and back the
// other way at 144 tiles of 256 (3072^3 881 vs 763, ragged 3000^3 780 vs
// 577) and at 256 (4096x4096x1024 964 vs 771).
constexpr int64_t SMALL_TILE_MAX = 128;

// Above that, 192 x 192 tiles when they fill the CUs' rounds better, by
// enough to pay for their lower rate: a 192-wide workgroup (96 x 96 per
// wave) reads a third more operand bytes per MFMA than a 256-wide one and
// runs at about 0.82 of its rate (0.72 in the range-checked form, on
// shapes 192 does not divide), measured at full rounds.  Each form is
// scored as rate x fill, fill = tiles / (rounds x 256 CUs), one workgroup
// per CU at either size.  Measured, bf16 TFLOP/s (256 -> 192): 3072^3
// 879 -> 1127, 6144^3 1130 -> 1232, ragged 3000^3 778 -> 920, 6144^2 x
// 2048 993 -> 1054, 3072^2 x 1024 707 -> 818; and the other way 3840^3
// 1254 vs 1020, 4608^3 970 vs 958, 5120^3 1199 vs 1015, 12288^2 x 1024
// 1087 vs 924.
constexpr int64_t CUS = 256;
constexpr double RATE_192 = 0.82, RATE_192_RAGGED = 0.72;

double round_fill(int64_t tiles)
{
    return static_cast<double>(tiles) / static_cast<double>(cdiv(tiles, CUS) * CUS);
}

bool prefer_192(const Call &c, int layout)
{
    if (!dma_any(c, layout, 1, 192))
        return false;
    const double r = dma_interior(c, layout, 1, 192) ? RATE_192 : RATE_192_RAGGED;
    return r * round_fill(cdiv(c.M, 192) * cdiv(c.N, 192)) >
           round_fill(cdiv(c.M, 256) * cdiv(c.N, 256));
}

// The rows of C at and below `row0` as a problem of their own (A's rows
// likewise; B whole).
Call lower_rows(const Call &c, int64_t row0)
{
    Call d = c;
    d.M = c.M - row0;
    d.A = static_cast<const char *>(c.A) + row0 * c.sam * item_size(c.in);
    d.C = static_cast<const char *>(c.C) + row0 * c.scm * item_size(c.out);
    return d;
}
Call upper_rows(const Call &c, int64_t rows)
{
    Call d = c;
    d.M = rows;
    return d;
}

// Split only the last, part-filled round of 256-wide tiles.  When the tiles
// do not fill whole rounds of the 256 CUs, the top tile-rows that do run
// unsplit and the remaining tile-rows, fewer than one round of tiles, run
// with K in S slices so that tiles x S nearly fills one more round; their
// fp32 partials are summed by the split-K pass.  Modelled in units of one
// chunk of K on one tile: unsplit rows ceil(tiles / 256) x chunks, the tail
// ceil(chunks / S), plus TAIL_PARTIAL_COST per partial tile written and read
// back (fitted to measurements: 0.22-0.33).  Taken when that beats the
// plain plan (256 or 192 wide) by 3%.  Measured, bf16 TFLOP/s (plain ->
// split tail): 4096 x 5120 x 4096 959 -> 1079-1095, 5120 x 4096 x 4096
// 954 -> 1110, 6000^3 1028 -> 1161, 7000^3 1049 -> 1212, 4096 x 5120 x 8192
// 1023 -> 1243; 6144^3 on 192-wide tiles 1232 against 1264.
constexpr double TAIL_PARTIAL_COST = 0.3;
constexpr int64_t TAIL_MAX_SPLIT = 16, TAIL_MIN_SLICE = 256;

bool pick_tail_split(const Call &c, int layout, int plain_tile, uint64_t ws_budget,
                     int64_t &dp_rows, int64_t &split)
{
    const int64_t gm = cdiv(c.M, 256), gn = cdiv(c.N, 256), tiles = gm * gn;
    if (tiles <= CUS || tiles % CUS == 0)
        return false;
    const int64_t rows_dp = (tiles / CUS) * CUS / gn;  // tile-rows in whole rounds
    if (rows_dp <= 0 || rows_dp >= gm)
        return false;
    const int64_t tail = (gm - rows_dp) * gn;
    const double nk = static_cast<double>(cdiv(c.K, 32));
    double plain = static_cast<double>(cdiv(tiles, CUS)) * nk;
    if (plain_tile == 192) {
        const double r = dma_interior(c, layout, 1, 192) ? RATE_192 : RATE_192_RAGGED;
        plain = static_cast<double>(cdiv(cdiv(c.M, 192) * cdiv(c.N, 192), CUS)) * nk *
                (192.0 * 192.0) / (256.0 * 256.0) / r;
    }
    const Call top = upper_rows(c, rows_dp * 256), low = lower_rows(c, rows_dp * 256);
    if (!dma_any(top, layout, 1, 256))
        return false;
    const double dp = static_cast<double>(cdiv(rows_dp * gn, CUS)) * nk;
    double best = 0.97 * plain;
    bool found = false;
    // fp32 partials of one slice of the split rows
    const uint64_t slice_bytes = static_cast<uint64_t>(low.M) * static_cast<uint64_t>(c.N) * 4u;
    for (int64_t S = 2; S <= TAIL_MAX_SPLIT && tail * S <= CUS; ++S) {
        if (static_cast<uint64_t>(S) > ws_budget / slice_bytes)
            break;
        if (c.K / S < TAIL_MIN_SLICE || !dma_any(low, layout, S, 256))
            continue;
        const double t = dp + std::ceil(nk / static_cast<double>(S)) +
                         TAIL_PARTIAL_COST * static_cast<double>(S * tail);
        if (t < best) {
            best = t;
            split = S;
            found = true;
        }
    }
    if (found)
        dp_rows = rows_dp * 256;
    return found;
}

// Split-K for problems whose 128 x 128 tiles still cannot fill the chip and
// whose K is long: up to S_max = min(256 / tiles, K / 2048) slices (slices of
// at least 2048, 64 pipelined chunks).  The largest power of two within
// that is taken when it reaches 3/4 of S_max (it usually divides K into
// whole chunks, the faster interior form), else S_max itself.  Measured
// (128 tiles; us): 1024x1024x8192 S=1 58, S=4 25, S=8 28; 512x512x65536
// fp16 S=8 63, S=16 42; 1024^3 S=1 faster than S=2; 768x768x32768 (36
// tiles) S=4 63, S=7 51; 384x384x65536 (9 tiles) S=16 37, S=28 32;
// 896x896x16384 (49 tiles) S=4 and S=5 level.
int64_t pick_split(const Call &c, int layout, int64_t tiles, int tile, int64_t cap)
{
    int64_t s_max = CUS / tiles;
    if (c.K / 2048 < s_max)
        s_max = c.K / 2048;
    if (cap < s_max)
        s_max = cap;
    if (s_max <= 1)
        return 1;
    int64_t p2 = 1;
    while (p2 * 2 <= s_max)
        p2 *= 2;
    if (4 * p2 < 3 * s_max && dma_any(c, layout, s_max, tile))
        return s_max;
    for (; p2 > 1; p2 /= 2)
        if (dma_any(c, layout, p2, tile))
            return p2;
    return 1;
}

// fp32 on the matrix cores: the tile (256, 192 or 128 wide) whose rounds
// over the CUs take the least time, each round priced against a round of
// 256-wide tiles (one workgroup per CU) over the same K.  From timings at
// 2048^3-8192^3 (the model's times are off by up to 16%, but it picked the
// fastest of the three tiles at every size tried): a round of 192-wide tiles
// (one per CU) costs 0.66; the interior 128-wide form runs one workgroup per
// CU at 0.273 a round, the range-checked one up to three, and a round with
// one, two or three of them per CU costs 0.273, 0.548 or 0.877.  4096^3 and
// 8192^3 take 256, 3000^3 192 (114 against 86 TFLOP/s on 128), 2048^3,
// 4608^3 and 6000^3 128.
constexpr double F32_ROUND_192 = 0.66;
constexpr double F32_ROUND_128[3] = {0.273, 0.548, 0.877};

int32_t f32_tile(const Call &c)
{
    const int64_t t256 = cdiv(c.M, 256) * cdiv(c.N, 256), t192 = cdiv(c.M, 192) * cdiv(c.N, 192);
    const int64_t t128 = cdiv(c.M, 128) * cdiv(c.N, 128);
    const double cost256 = static_cast<double>(cdiv(t256, CUS));
    const double cost192 = static_cast<double>(cdiv(t192, CUS)) * F32_ROUND_192;
    const bool interior128 = c.M % 128 == 0 && c.N % 128 == 0 && c.K % 16 == 0;
    const int64_t rem = t128 % (3 * CUS);
    const double cost128 =
        interior128 ? static_cast<double>(cdiv(t128, CUS)) * F32_ROUND_128[0]
                    : static_cast<double>(t128 / (3 * CUS)) * F32_ROUND_128[2] +
                          (rem == 0 ? 0.0 : F32_ROUND_128[cdiv(rem, CUS) - 1]);
    if (cost256 <= cost192 && cost256 <= cost128)
        return 256;
    return cost192 < cost128 ? 192 : 128;
}

// fp32 chunk depth: 32 at 256 x 256 when K is a multiple of 32 (one barrier
// and one refill round per 32 k; 4096^3 and 8192^3 about 1% faster, in 144
// KiB of LDS), else 16 -- a K off 32 would send every chunk through the
// range-checked loads.  192 x 192 always takes 32 (at 16 an operand tile is
// an odd number of 16-byte units per thread); 128 x 128 keeps 16 (32 there
// leaves the range-checked form two workgroups per CU instead of three and
// cost it 5% at 3000^3).
int32_t f32_block_k(const Call &c, int32_t tile)
{
    return tile == 192 || (tile == 256 && c.K % 32 == 0) ? 32 : 16;
}

// The pipelined kernel's interior form at tile 256 runs with 4 waves of
// 128 x 128 (one per SIMD) when each tile's K loop is at least this long,
// else with 8 waves of 128 x 64 (two per SIMD, which cover each other's
// waits).  A 4-wave wave reads a third less LDS per MFMA, and on this
// power-limited chip that shows as clock.  Side by side (bf16 unless noted,
// TFLOP/s, 8 -> 4 waves): K = 4096 and up gained 0.7-3.8% (fp16 4096^3
// 1160 -> 1204, 8192^3 1347 -> 1364, 6144^3, 5120^3) except 8192 x 4096 x
// 4096 (1313 -> 1295); K = 1024 lost (4096 x 4096 x 1024 966 -> 948,
// 16384 x 16384 x 1024 1068 -> 885).  With the paired stages, K = 2048 still
// favours 8 waves (8192^2 x 2048 NN +2.8%, NT +1.2%) and K = 3072 4 waves
// (fp16 8192^2 x 3072 -> fp32 +4.6%, 6144^2 x 3072 level).  The
// range-checked form has 8 waves.
#ifndef DTM_FOUR_WAVE_MIN_K
#define DTM_FOUR_WAVE_MIN_K 3072
#endif
constexpr int64_t FOUR_WAVE_MIN_K = DTM_FOUR_WAVE_MIN_K;

// The wave-K kernel (128 x 128 tiles whose 4 waves split the K loop, each
// wave holding the whole tile) takes over from the 128-wide pipelined tile
// when each tile's K loop (per slice when split) is 4096 or more.  Measured
// side by side (us, wave-K against 4 waves of 64 x 64, bf16 / fp16 -> fp32
// pairs): loops of 8192 and more gain 8-17% (2048^2 x 8192 61.4 / 69.3,
// 2048^2 x 16384 113.3 / 129.1, 1536^2 x 8192 55.6 / 63.7, 8192 x 1024 x
// 8192 121.6 / 134.6, 1024^2 x 32768 split 4 65.3 / 71.3), loops of 4096 gain
// 2-10% whether or not the workgroups fill the 256 CUs (512^2 x 65536 split 16
// 41.7 / 42.3, 1024^2 x 16384 split 4 40.3 / 41.2, 640^2 x 32768 split 8 35.6
// / 37.7, 896^2 x 16384 split 4 35.4 / 38.1, 1536^2 x 4096 32.9 / 36.3), and
// loops of 2048 lose 1-8% (1024^2 x 8192 split 4 27.2 / 26.3, 2048^3 24.2 /
// 22.4, 256^2 x 65536 split 32 25.2 / 24.5).
constexpr int64_t WAVEK_MIN_K = 4096;  // K loop per tile (per slice when split)

bool prefer_wavek(const Call &c, int layout, int64_t splits)
{
    return wavek_fits(c, layout, splits) && c.K / splits >= WAVEK_MIN_K;
}

// The plan for a call.  ws_budget: bytes of workspace the call can use;
// the selector splits K only as far as its partials fit in it (UINT64_MAX:
// no limit).  A forced split is not capped; run() then checks the workspace.
int make_plan(const Call &c, const dtm_tile_config *force, uint64_t ws_budget, dtm_plan *out)
{
    if (!out)
        return DTM_ERR_NULL_POINTER;
    std::memset(out, 0, sizeof(*out));
    const int st = validate(c);
    if (st != DTM_OK)
        return st;
    dtm_plan p;
    std::memset(&p, 0, sizeof(p));
    p.split_k = 1;
    if (c.M == 0 || c.N == 0) {
        p.kernel = DTM_KERNEL_NONE;
        *out = p;
        return DTM_OK;
    }
    // Every MFMA kernel reads all four operand layouts.
    const int layout = mfma_layout(c);
    const bool dma = c.K > 0 && dma_any(c, layout, 1);  // the pipelined kernel, either form
    // views off 16-byte boundaries: the register-staged kernel only
    const int layout16u = layout < 0 ? mfma16_unaligned_layout(c) : -1;
    const bool fast16 = is16(c) && (layout >= 0 || layout16u >= 0);
    const int layout32 = c.in == DTM_F32 ? mfma32_layout(c, nullptr) : -1;
    const bool fast32 = layout32 >= 0;
    p.fast_path = fast16 || fast32 ? 1 : 0;
    if (c.K == 0) {
        p.kernel = DTM_KERNEL_ZERO_FILL;
        p.block_m = p.block_n = p.block_k = 1;
        p.threads = 256;
        p.grid_m = c.M;
        p.grid_n = c.N;
        *out = p;
        return DTM_OK;
    }

    const bool forced_dims = force && (force->block_m || force->block_n || force->block_k);
    const int64_t forced_split = force && force->split_k > 1 ? force->split_k : 0;
    int kernel = force && force->kernel
                     ? force->kernel
                     : (fast16 ? DTM_KERNEL_MFMA_F16 : fast32 ? DTM_KERNEL_MFMA_F32
                                                              : DTM_KERNEL_GENERIC);
    if (kernel == DTM_KERNEL_MFMA_F16) {
        if (!fast16)
            return DTM_ERR_CONFIG;
        if (forced_dims) {
            const bool dma_cfg = is_dma_tile(force->block_m, force->block_n, force->block_k);
            if (dma_cfg ? !(c.K > 0 && dma_any(c, layout, 1, force->block_m))
                        : !dtm::mfma16_has_config(force->block_m, force->block_n, force->block_k))
                return DTM_ERR_CONFIG;
            p.block_m = force->block_m;
            p.block_n = force->block_n;
            p.block_k = force->block_k;
        } else {
            // The pipelined kernel whenever it can run the problem (measured
            // ahead of the register-staged kernel at every tile count): with
            // 128-wide tiles, and split-K when even those are few and K is
            // long, when the 256-wide tiles are few; with 192-wide tiles when
            // they fill the CUs better; otherwise the register-staged kernel.
            const int64_t tiles256 = cdiv(c.M, 256) * cdiv(c.N, 256);
            if (dma) {
                const int tile = tiles256 <= SMALL_TILE_MAX && dma_any(c, layout, 1, 128) ? 128
                                 : prefer_192(c, layout)                                 ? 192
                                                                                         : 256;
                p.block_m = p.block_n = tile;
                p.block_k = 32;
                const uint64_t slice_bytes =
                    static_cast<uint64_t>(c.M) * static_cast<uint64_t>(c.N) * 4u;
                const uint64_t cap = ws_budget / slice_bytes;
                p.split_k = tile == 128 ? static_cast<int32_t>(pick_split(
                                              c, layout, cdiv(c.M, 128) * cdiv(c.N, 128), 128,
                                              cap < CUS ? static_cast<int64_t>(cap) : CUS))
                                        : 1;
                int64_t dp_rows = 0, tail_split = 1;
                if (tile != 128 &&
                    pick_tail_split(c, layout, tile, ws_budget, dp_rows, tail_split)) {
                    p.block_m = p.block_n = 256;
                    p.split_k = static_cast<int32_t>(tail_split);
                    p.dp_rows = dp_rows;
                }
            } else {
                p.block_m = p.block_n = tiles256 >= 256 ? 256 : 128;
                p.block_k = 64;
            }
        }
        if (forced_split) {
            // split-K runs on the pipelined kernel only
            if (!is_dma_tile(p.block_m, p.block_n, p.block_k) ||
                !dma_any(c, layout, forced_split, p.block_m))
                return DTM_ERR_CONFIG;
            p.split_k = static_cast<int32_t>(forced_split);
            p.dp_rows = 0;
        }
        if (force && force->dp_rows) {
            // unsplit top rows: whole tiles, below M, each part runnable
            const int64_t r = force->dp_rows;
            if (!forced_split || r < 0 || r % p.block_m || r >= c.M ||
                !dma_any(upper_rows(c, r), layout, 1, p.block_m) ||
                !dma_any(lower_rows(c, r), layout, forced_split, p.block_m))
                return DTM_ERR_CONFIG;
            p.dp_rows = r;
        }
        p.threads = 256;  // the pipelined kernel's is settled below
        p.layout = layout >= 0 ? layout : layout16u;
    } else if (kernel == DTM_KERNEL_MFMA_F16_WAVEK) {
        // forced only: 128 x 128 x 32 tiles, 4 waves, the forced split or none
        const int64_t S = forced_split ? forced_split : 1;
        if (!fast16 || !wavek_fits(c, layout, S) || force->dp_rows ||
            (forced_dims &&
             (force->block_m != 128 || force->block_n != 128 || force->block_k != 32)) ||
            (force->threads && force->threads != 256))
            return DTM_ERR_CONFIG;
        p.block_m = p.block_n = 128;
        p.block_k = 32;
        p.split_k = static_cast<int32_t>(S);
        p.threads = 256;
        p.layout = layout;
    } else if (kernel == DTM_KERNEL_MFMA_F32) {
        if (!fast32)
            return DTM_ERR_CONFIG;
        if (forced_dims && !dtm::mfma32_has_config(force->block_m, force->block_n, force->block_k))
            return DTM_ERR_CONFIG;
        p.block_m = p.block_n = forced_dims ? force->block_m : f32_tile(c);
        p.block_k = forced_dims ? force->block_k : f32_block_k(c, p.block_m);
        p.threads = 256;
        p.layout = layout32;
    } else if (kernel == DTM_KERNEL_GENERIC || kernel == DTM_KERNEL_GENERIC_FP16ACC) {
        if (kernel == DTM_KERNEL_GENERIC_FP16ACC && c.in != DTM_F16)
            return DTM_ERR_CONFIG;
        if (forced_dims) {
            if (!dtm::generic_has_config(force->block_m, force->block_n, force->block_k))
                return DTM_ERR_CONFIG;
            p.block_m = force->block_m;
            p.block_n = force->block_n;
            p.block_k = force->block_k;
        } else {
            pick_generic(c, p);
        }
        p.threads = dtm::generic_threads(p.block_m, p.block_n, p.block_k);
    } else {
        return DTM_ERR_CONFIG;
    }
    // the selector's own 128-wide plans: the wave-K kernel where it pays
    if (kernel == DTM_KERNEL_MFMA_F16 && !(force && (force->kernel || force->split_k > 1 ||
                                                     force->dp_rows || force->threads)) &&
        !forced_dims && p.block_m == 128 && p.block_k == 32 && p.dp_rows == 0 &&
        prefer_wavek(c, layout, p.split_k))
        kernel = DTM_KERNEL_MFMA_F16_WAVEK;
    if ((forced_split || (force && force->dp_rows)) && kernel != DTM_KERNEL_MFMA_F16 &&
        kernel != DTM_KERNEL_MFMA_F16_WAVEK)
        return DTM_ERR_CONFIG;
    p.kernel = kernel;
    fill_grid(c, p);
    if (kernel == DTM_KERNEL_MFMA_F16 && layout < 0)
        p.ragged = 1;  // views off 16-byte boundaries: the range-checked form
    const bool dma_tile = kernel == DTM_KERNEL_MFMA_F16 && p.block_k == 32;
    if (dma_tile) {
        // which form of the pipelined kernel, and how many waves (with
        // unsplit top rows: ragged when either part is; the top part's waves)
        bool top_ragged = !dma_interior(c, layout, p.split_k, p.block_m);
        bool low_ragged = top_ragged;
        if (p.dp_rows > 0) {
            top_ragged = !dma_interior(upper_rows(c, p.dp_rows), layout, 1, p.block_m);
            low_ragged = !dma_interior(lower_rows(c, p.dp_rows), layout, p.split_k, p.block_m);
        }
        p.ragged = top_ragged || low_ragged ? 1 : 0;
        const int forced_threads = force ? force->threads : 0;
        if (forced_threads) {
            if (forced_threads % 64 ||
                !dtm::mfma16_dma_waves_ok(p.block_m, forced_threads / 64, top_ragged) ||
                !dtm::mfma16_dma_waves_ok(p.block_m, forced_threads / 64, low_ragged))
                return DTM_ERR_CONFIG;
            p.threads = forced_threads;
        } else if (p.block_m != 256) {
            p.threads = 256;  // 192 and 128: 4 waves
        } else {
            const int64_t kloop = (p.dp_rows > 0 ? cdiv(c.K, p.block_k) : p.k_iters) * p.block_k;
            p.threads = !top_ragged && kloop >= FOUR_WAVE_MIN_K ? 256 : 512;
        }
    } else if (force && force->threads && kernel != DTM_KERNEL_MFMA_F16_WAVEK) {
        return DTM_ERR_CONFIG;  // a workgroup size is chosen for the pipelined kernels only
    }
    if (p.split_k > 1)
        p.workspace_bytes = static_cast<uint64_t>(p.split_k) *
                            static_cast<uint64_t>(c.M - p.dp_rows) *
                            static_cast<uint64_t>(c.N) * sizeof(float);
    if (p.grid_m * p.grid_n > 0x7fffffffLL)
        return DTM_ERR_CONFIG;
    *out = p;
    return DTM_OK;
}

// ---- device check ---------------------------------------------------------

// With pointer checks on: every view the plan touches (A and B when K > 0,
// C, a caller's workspace) inside one device allocation of this device.
int check_pointers(const Call &c, const dtm_plan &p, const void *workspace)
{
    auto view = [](const void *base, int64_t rows, int64_t cols, int64_t sr, int64_t sc,
                   int64_t item) {
        uintptr_t lo, hi;
        if (!view_range(base, rows, cols, sr, sc, item, lo, hi))
            return static_cast<int>(DTM_ERR_POINTER);
        return dtm::check_view_memory(lo, hi);
    };
    int st = view(c.C, c.M, c.N, c.scm, c.scn, item_size(c.out));
    if (st == DTM_OK && c.K > 0)
        st = view(c.A, c.M, c.K, c.sam, c.sak, item_size(c.in));
    if (st == DTM_OK && c.K > 0)
        st = view(c.B, c.K, c.N, c.sbk, c.sbn, item_size(c.in));
    if (st == DTM_OK && workspace && p.workspace_bytes > 0) {
        const uintptr_t w = reinterpret_cast<uintptr_t>(workspace);
        st = dtm::check_view_memory(w, w + p.workspace_bytes);
    }
    return st;
}

// Launch a validated plan; `ws` is the split-K workspace when split_k > 1.
int launch_plan(const Call &c, const dtm_plan &p, void *ws, hipStream_t s)
{
    GemmArgs a{c.M, c.N, c.K, c.A, c.sam, c.sak, c.B, c.sbk, c.sbn, const_cast<void *>(c.C),
               c.scm, c.scn};
    hipError_t e = hipSuccess;
    switch (p.kernel) {
    case DTM_KERNEL_ZERO_FILL: e = dtm::launch_zero_fill(a, c.out, s); break;
    case DTM_KERNEL_GENERIC:
        e = dtm::launch_generic(a, c.in, c.out, p.block_m, p.block_n, p.block_k, s);
        break;
    case DTM_KERNEL_GENERIC_FP16ACC:
        e = dtm::launch_generic_fp16acc(a, c.out, p.block_m, p.block_n, p.block_k, s);
        break;
    case DTM_KERNEL_MFMA_F16:
        if (p.split_k > 1) {
            e = dtm::launch_mfma16_dma_partials(a, c.in, p.layout, p.split_k, p.ragged != 0,
                                                 a_view_bytes(c), b_view_bytes(c), p.block_m,
                                                 p.threads / 64, static_cast<float *>(ws), s);
            if (e == hipSuccess)
                e = dtm::launch_splitk_reduce(a, c.out, p.split_k, static_cast<float *>(ws), s);
        } else if (p.block_k == 32 && p.ragged)
            e = dtm::launch_mfma16_dma_ragged(a, c.in, c.out, p.layout, a_view_bytes(c),
                                              b_view_bytes(c), p.block_m, p.threads / 64, s);
        else if (p.block_k == 32)
            e = dtm::launch_mfma16_dma(a, c.in, c.out, p.layout, p.block_m, p.threads / 64, s);
        else
            e = dtm::launch_mfma16(a, c.in, c.out, p.block_m, p.block_n, p.block_k, p.layout,
                                   p.ragged != 0, s);
        break;
    case DTM_KERNEL_MFMA_F16_WAVEK:
        if (p.split_k > 1) {
            e = dtm::launch_mfma16_wavek_partials(a, c.in, p.layout, p.split_k,
                                                  static_cast<float *>(ws), s);
            if (e == hipSuccess)
                e = dtm::launch_splitk_reduce(a, c.out, p.split_k, static_cast<float *>(ws), s);
        } else {
            e = dtm::launch_mfma16_wavek(a, c.in, c.out, p.layout, s);
        }
        break;
    case DTM_KERNEL_MFMA_F32: {
        bool aligned = false;
        mfma32_layout(c, &aligned);
        e = dtm::launch_mfma32(a, c.out, p.block_m, p.block_n, p.block_k, p.layout,
                               p.ragged != 0, aligned, s);
        break;
    }
    default: return DTM_ERR_CONFIG;
    }
    return e == hipSuccess ? DTM_OK : DTM_ERR_LAUNCH;
}

// The workspace a call can use: the caller's (gemm_ex) or what is reserved
// for the stream, capped by a forced workspace_limit.
uint64_t call_budget(const dtm_tile_config *force, uint64_t available)
{
    const uint64_t limit = force && force->workspace_limit ? force->workspace_limit : UINT64_MAX;
    return available < limit ? available : limit;
}

// library_ws: `workspace` is memory of the library's own (the pointer
// checks leave it out).
int run(const Call &c, const dtm_tile_config *force, void *workspace, uint64_t workspace_bytes,
        void *stream, bool library_ws = false)
{
    // Without a caller's workspace, the one reserved for this stream (if
    // any) bounds the plan; the lease is held until every launch of this
    // call is queued.
    if (!dtm::resolve_force(force))
        return DTM_ERR_CONFIG;
    std::optional<dtm::WorkspaceLease> lease;
    if (!workspace)
        lease.emplace(stream);
    void *ws = workspace ? workspace : lease->ptr();
    const uint64_t ws_bytes = workspace ? workspace_bytes : lease->bytes();
    dtm_plan p;
    int st = make_plan(c, force, call_budget(force, ws_bytes), &p);
    if (st != DTM_OK)
        return st;
    if (p.kernel == DTM_KERNEL_NONE)
        return DTM_OK;
    st = check_device();
    if (st != DTM_OK)
        return st;
    if (dtm::pointer_checks_on()) {
        st = check_pointers(c, p, library_ws ? nullptr : workspace);
        if (st != DTM_OK)
            return st;
    }
    if (p.split_k > 1) {
        if (!ws || ws_bytes < p.workspace_bytes || (reinterpret_cast<uintptr_t>(ws) & 15))
            return DTM_ERR_WORKSPACE;
    } else {
        ws = nullptr;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.dp_rows == 0)
        return launch_plan(c, p, ws, s);
    // Unsplit top rows, then the split rows below them, in stream order.
    const Call top = upper_rows(c, p.dp_rows), low = lower_rows(c, p.dp_rows);
    const int32_t threads = force ? force->threads : 0;
    const dtm_tile_config f_top{DTM_KERNEL_MFMA_F16, p.block_m, p.block_n, p.block_k, 1, threads,
                                0, 0};
    const dtm_tile_config f_low{DTM_KERNEL_MFMA_F16, p.block_m, p.block_n, p.block_k, p.split_k,
                                threads, 0, 0};
    dtm_plan p_top, p_low;
    st = make_plan(top, &f_top, UINT64_MAX, &p_top);
    if (st == DTM_OK)
        st = make_plan(low, &f_low, UINT64_MAX, &p_low);
    if (st != DTM_OK)
        return st;
    st = launch_plan(top, p_top, nullptr, s);
    return st == DTM_OK ? launch_plan(low, p_low, ws, s) : st;
}

}  // namespace

namespace dtm {

int gemm_ex_library_ws(int64_t M, int64_t N, int64_t K, const void *A, int64_t sam, int64_t sak,
                       const void *B, int64_t sbk, int64_t sbn, void *C, int64_t scm, int64_t scn,
                       int in_dtype, int out_dtype, const dtm_tile_config *force, void *ws,
                       uint64_t ws_bytes, void *stream)
{
    const Call c{M, N, K, A, sam, sak, B, sbk, sbn, C, scm, scn, in_dtype, out_dtype};
    return run(c, force, ws, ws_bytes, stream, true);
}

}  // namespace dtm

extern "C" {

int gemm(int64_t M, int64_t N, int64_t K, const void *A, int64_t stride_am, int64_t stride_ak,
         const void *B, int64_t stride_bk, int64_t stride_bn, void *C, int64_t stride_cm,
         int64_t stride_cn, int in_dtype, int out_dtype, void *stream)
{
    const Call c{M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                 stride_cn, in_dtype, out_dtype};
    return run(c, nullptr, nullptr, 0, stream);
}

int gemm_plan(int64_t M, int64_t N, int64_t K, const void *A, int64_t stride_am,
              int64_t stride_ak, const void *B, int64_t stride_bk, int64_t stride_bn,
              const void *C, int64_t stride_cm, int64_t stride_cn, int in_dtype, int out_dtype,
              const dtm_tile_config *force, dtm_plan *out)
{
    const Call c{M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                 stride_cn, in_dtype, out_dtype};
    if (!dtm::resolve_force(force))
        return DTM_ERR_CONFIG;
    return make_plan(c, force, call_budget(force, UINT64_MAX), out);
}

int gemm_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t stride_am, int64_t stride_ak,
            const void *B, int64_t stride_bk, int64_t stride_bn, void *C, int64_t stride_cm,
            int64_t stride_cn, int in_dtype, int out_dtype, const dtm_tile_config *force,
            void *workspace, uint64_t workspace_bytes, void *stream)
{
    const Call c{M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C, stride_cm,
                 stride_cn, in_dtype, out_dtype};
    return run(c, force, workspace, workspace_bytes, stream);
}

const char *gemm_status_string(int status)
{
    switch (status) {
    case DTM_OK: return "ok";
    case DTM_ERR_INVALID_DIM: return "invalid dimension: M, N and K must be in [0, 2^31)";
    case DTM_ERR_NULL_POINTER: return "null pointer for an operand or out-parameter that is needed";
    case DTM_ERR_DTYPE: return "unknown dtype code (expected DTM_F32, DTM_F16 or DTM_BF16)";
    case DTM_ERR_STRIDE:
        return "bad C strides (negative, or two elements of C overlap) or a view whose address "
               "range overflows";
    case DTM_ERR_ALIAS: return "C overlaps A or B";
    case DTM_ERR_CONFIG: return "forced tile configuration is not available for this problem";
    case DTM_ERR_WORKSPACE:
        return "workspace smaller than the plan needs (reserve one with gemm_workspace_reserve "
               "or pass a larger one), or its reservation failed";
    case DTM_ERR_DEVICE: return "current HIP device is not gfx950 or could not be queried";
    case DTM_ERR_LAUNCH: return "kernel launch failed";
    case DTM_ERR_POINTER:
        return "pointer check: a view is not inside one device allocation of the current device";
    case DTM_ERR_SCRATCH:
        return "the plan needs more scratch than gemm_ex_noalloc's fixed device array holds "
               "(use gemm_ex with a workspace, or a smaller split)";
    }
    return "unknown status";
}

const char *gemm_kernel_name(int kernel)
{
    switch (kernel) {
    case DTM_KERNEL_NONE: return "none";
    case DTM_KERNEL_ZERO_FILL: return "zero_fill";
    case DTM_KERNEL_GENERIC: return "generic";
    case DTM_KERNEL_MFMA_F16: return "mfma_f16";
    case DTM_KERNEL_MFMA_F32: return "mfma_f32";
    case DTM_KERNEL_GENERIC_FP16ACC: return "generic_fp16acc";
    case DTM_KERNEL_MFMA_F16_WAVEK: return "mfma_f16_wavek";
    }
    return "unknown";
}

int gemm_mfma_probe(int in_dtype, int layout, int paired, const void *A, const void *B, void *C,
                    void *stream)
{
    if (in_dtype != DTM_F16 && in_dtype != DTM_BF16)
        return DTM_ERR_DTYPE;
    if (layout < 0 || layout > (DTM_LAYOUT_A_M_CONTIG | DTM_LAYOUT_B_K_CONTIG) ||
        (paired != 0 && paired != 1))
        return DTM_ERR_CONFIG;
    if (!A || !B || !C)
        return DTM_ERR_NULL_POINTER;
    if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B) |
         reinterpret_cast<uintptr_t>(C)) & 15)
        return DTM_ERR_STRIDE;
    const int st = check_device();
    if (st != DTM_OK)
        return st;
    const hipError_t e = dtm::launch_mfma_probe(in_dtype, layout, paired != 0, A, B,
                                                static_cast<float *>(C),
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DTM_OK : DTM_ERR_LAUNCH;
}

int gemm_set_pointer_checks(int on)
{
    return dtm::g_pointer_checks.exchange(on != 0) ? 1 : 0;
}

}  // extern "C"
