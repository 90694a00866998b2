// ssu_api.hip -- the C ABI declared in include/ssu.h: host-side validation,
// launch-shape selection and the single kernel launch. Validation reads only the
// argument struct (sizes, dtypes, null-ness, alignment, address ranges); it never
// touches device memory, so a rejected call costs no HIP call at all.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "ssu.h"
#include "ssu_launch.h"

namespace {

thread_local char t_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_error, sizeof(t_error), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    t_error[0] = '\0';
    return SSU_OK;
}

}  // namespace

int ssu::report(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_error, sizeof(t_error), fmt, ap);
    va_end(ap);
    return code;
}

int ssu::report_ok() { return ok(); }

namespace {

bool log_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("SSU_LOG");
        return v && v[0] && std::strcmp(v, "0") != 0;
    }();
    return on;
}

size_t dtype_size(int32_t d) { return d == SSU_F32 ? 4 : 2; }
bool is_dtype(int32_t d) { return d == SSU_F32 || d == SSU_F16 || d == SSU_BF16; }
bool is_index(int32_t d) { return d == SSU_I32 || d == SSU_I64; }
const char* dtype_name(int32_t d) {
    return d == SSU_F32 ? "fp32" : d == SSU_F16 ? "fp16" : d == SSU_BF16 ? "bf16" : "?";
}

struct Range {
    const char* name;
    const void* p;
    size_t bytes;
};

bool overlaps(const Range& a, const Range& b) {
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const auto a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Checks shared by both entry points. `rows` rows of x/out/B/C/z/dt are used.
int check_operands(const ssu_operands& op, int64_t rows, bool work, bool packed) {
    if (!is_dtype(op.state_dtype))
        return fail(SSU_ERR_INVALID_ARGUMENT, "state_dtype %d is not an ssu_dtype", op.state_dtype);
    if (!is_dtype(op.io_dtype))
        return fail(SSU_ERR_INVALID_ARGUMENT, "io_dtype %d is not an ssu_dtype", op.io_dtype);
    if (op.nslots < 1 || op.nheads < 1 || op.headdim < 1 || op.dstate < 1 || op.ngroups < 1)
        return fail(SSU_ERR_INVALID_ARGUMENT,
                    "sizes must be positive: nslots=%lld nheads=%lld headdim=%lld dstate=%lld "
                    "ngroups=%lld",
                    (long long)op.nslots, (long long)op.nheads, (long long)op.headdim,
                    (long long)op.dstate, (long long)op.ngroups);
    if (op.nheads % op.ngroups != 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "nheads (%lld) must be a multiple of ngroups (%lld)",
                    (long long)op.nheads, (long long)op.ngroups);
    if (op.dt_per_dim != 0 && op.dt_per_dim != 1)
        return fail(SSU_ERR_INVALID_ARGUMENT, "dt_per_dim must be 0 or 1, got %d", op.dt_per_dim);
    const int64_t hpg = op.nheads / op.ngroups;
    const int32_t hpb = op.heads_per_block;
    if (hpb != 0 && hpb != 1 && hpb != 2 && hpb != 4)
        return fail(SSU_ERR_INVALID_ARGUMENT, "heads_per_block must be 0, 1, 2 or 4, got %d", hpb);
    if (hpb > 1 && hpg % hpb != 0)
        return fail(SSU_ERR_INVALID_ARGUMENT,
                    "heads_per_block (%d) must divide nheads / ngroups (%lld)", hpb, (long long)hpg);
    if (op.philox_rounds < 0 || op.philox_rounds > 64)
        return fail(SSU_ERR_INVALID_ARGUMENT, "philox_rounds must be in [0, 64], got %d",
                    op.philox_rounds);
    if (op.tile_order < 0 || op.tile_order > 3)
        return fail(SSU_ERR_INVALID_ARGUMENT, "tile_order must be 0, 1, 2 or 3, got %d",
                    op.tile_order);
    if (op.loads_per_lane != 0 && op.loads_per_lane != 2 && op.loads_per_lane != 4)
        return fail(SSU_ERR_INVALID_ARGUMENT, "loads_per_lane must be 0, 2 or 4, got %d",
                    op.loads_per_lane);
    const int64_t N = op.dstate;
    if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256)
        return fail(SSU_ERR_UNSUPPORTED, "dstate %lld is not built (16, 32, 64, 128, 256 are)",
                    (long long)N);
    const int hmax = ssu::max_heads_per_block(static_cast<int>(N), packed);
    if (hpb > hmax)
        return fail(SSU_ERR_UNSUPPORTED, "heads_per_block %d exceeds %d for dstate %lld%s", hpb,
                    hmax, (long long)N, packed ? " (packed)" : "");
    const size_t ssz = dtype_size(op.state_dtype), iosz = dtype_size(op.io_dtype);
    if (op.nheads > INT32_MAX || op.headdim > INT32_MAX ||
        static_cast<uint64_t>(op.headdim) * N * ssz > 0x7fffffffull)
        return fail(SSU_ERR_UNSUPPORTED, "one head of one slot exceeds 2 GiB");
    if (!work) return SSU_OK;

    struct Req {
        const char* name;
        const void* p;
    } req[] = {{"state", op.state}, {"x", op.x}, {"B", op.B}, {"C", op.C},
               {"out", op.out},     {"dt", op.dt}, {"A", op.A}};
    for (const auto& q : req)
        if (!q.p) return fail(SSU_ERR_INVALID_ARGUMENT, "%s must not be NULL", q.name);
    if (reinterpret_cast<uintptr_t>(op.state) % 16 != 0)
        return fail(SSU_ERR_UNSUPPORTED, "state must be 16-byte aligned");
    struct Aligned {
        const char* name;
        const void* p;
        size_t a;
    } al[] = {{"x", op.x, iosz},  {"B", op.B, iosz},   {"C", op.C, iosz}, {"z", op.z, iosz},
              {"out", op.out, iosz}, {"dt", op.dt, 4}, {"A", op.A, 4},    {"D", op.D, 4},
              {"dt_bias", op.dt_bias, 4}, {"rand_seed", op.rand_seed, 8}};
    for (const auto& q : al)
        if (q.p && reinterpret_cast<uintptr_t>(q.p) % q.a != 0)
            return fail(SSU_ERR_INVALID_ARGUMENT, "%s is not aligned to its element size", q.name);

    const size_t H = op.nheads, P = op.headdim, G = op.ngroups, R = rows;
    const Range out{"out", op.out, R * H * P * iosz};
    const Range others[] = {
        {"x", op.x, R * H * P * iosz},
        {"z", op.z, R * H * P * iosz},
        {"B", op.B, R * G * N * iosz},
        {"C", op.C, R * G * N * iosz},
        {"dt", op.dt, R * H * (op.dt_per_dim ? P : 1) * 4},
        {"A", op.A, H * 4},
        {"D", op.D, H * 4},
        {"dt_bias", op.dt_bias, H * 4},
        {"state", op.state, static_cast<size_t>(op.nslots) * H * P * N * ssz},
    };
    for (const auto& o : others)
        if (overlaps(out, o)) return fail(SSU_ERR_INVALID_ARGUMENT, "out overlaps %s", o.name);
    return SSU_OK;
}

// Default launch shape. Measured on MI355X at the named decode shapes (dstate
// 128, headdim 64): a read+write one-token call streams best in small tiles
// (2 loads per lane, 2 heads per workgroup with an fp32 state, 1 with a 16-bit
// one); a read-only call in larger ones (4 loads per lane, 1 head per
// workgroup), and so the packed call, which writes several states per state
// read (4 loads per lane, 2 heads per workgroup). Tile
// order: varlen packed calls let each XCD take an equal contiguous share of
// every sequence's tiles (a block of its heads), which balances sequences of
// unequal token counts over the XCDs (3 % faster than contiguous ranges of
// sequences); one-token calls do so when that share is large (at least 256 KiB
// of state per sequence and XCD: 1-2 % faster at 80-128 heads of 64 x 128 fp32)
// and otherwise, like packed calls without cu_seqlens, let each XCD walk a
// contiguous range of tiles (smaller states stream better in longer runs).
struct Shape {
    int heads_per_block, loads_per_lane, xcd_order;  // xcd_order as in ssu::KernelParams
};

Shape default_shape(const ssu_operands& op, bool packed, bool equal_lengths) {
    const bool read_only = op.disable_state_update != 0;
    Shape s;
    const bool sr = op.rand_seed && op.state_dtype != SSU_F32 && !read_only;
    // Bytes of one sequence's state each XCD streams under per-sequence shares.
    const int64_t share = op.nheads * op.headdim * op.dstate * (op.state_dtype == SSU_F32 ? 4 : 2) /
                          ssu::kXcds;
    const int one_token_order = share >= (256 << 10) ? 2 : 1;
    if (packed)
        s = {2, 4, equal_lengths ? 1 : 2};
    else if (read_only)
        s = {1, 4, one_token_order};
    else if (sr)  // the Philox work of stochastic rounding wants bigger tiles
        s = {1, 4, one_token_order};
    else
        s = {op.state_dtype == SSU_F32 ? 2 : 1, 2, one_token_order};
    const int64_t hpg = op.nheads / op.ngroups;
    const int hmax = ssu::max_heads_per_block(static_cast<int>(op.dstate), packed);
    while (s.heads_per_block > 1 && (hpg % s.heads_per_block != 0 || s.heads_per_block > hmax))
        s.heads_per_block /= 2;
    return s;
}

void fill_common(ssu::KernelParams& k, const ssu_operands& op, bool packed,
                 bool equal_lengths) {
    k.state = op.state;
    k.x = op.x;
    k.B = op.B;
    k.C = op.C;
    k.z = op.z;
    k.out = op.out;
    k.dt = op.dt;
    k.A = op.A;
    k.D = op.D;
    k.dt_bias = op.dt_bias;
    // Stochastic rounding only changes 16-bit stores.
    k.rand_seed = op.state_dtype == SSU_F32 ? nullptr : static_cast<const int64_t*>(op.rand_seed);
    k.philox_rounds = op.philox_rounds ? op.philox_rounds : 10;
    k.nslots = op.nslots;
    k.pad_slot_id = op.pad_slot_id;
    k.nheads = static_cast<int32_t>(op.nheads);
    k.headdim = static_cast<int32_t>(op.headdim);
    k.ngroups = static_cast<int32_t>(op.ngroups);
    k.heads_per_group = static_cast<int32_t>(op.nheads / op.ngroups);
    const Shape dflt = default_shape(op, packed, equal_lengths);
    k.heads_per_block = op.heads_per_block ? op.heads_per_block : dflt.heads_per_block;
    k.loads_per_lane = op.loads_per_lane ? op.loads_per_lane : dflt.loads_per_lane;
    // tile_order 1: contiguous ranges, 2: hardware order, 3: per-sequence shares.
    k.xcd_order = op.tile_order == 0 ? dflt.xcd_order
                                     : (op.tile_order == 1 ? 1 : (op.tile_order == 3 ? 2 : 0));
    k.head_blocks = k.nheads / k.heads_per_block;
    k.dt_per_dim = op.dt_per_dim;
    k.dt_softplus = op.dt_softplus ? 1 : 0;
    k.disable_state_update = op.disable_state_update ? 1 : 0;
}

int launch(const ssu::KernelParams& k, const ssu_operands& op, int64_t nseq, void* stream,
           const char* entry) {
    const auto s = static_cast<hipStream_t>(stream);
    const int io = op.io_dtype, N = static_cast<int>(op.dstate);
    ssu::LaunchShape shape;
    hipError_t e;
    switch (op.state_dtype) {
        case SSU_F32: e = ssu::launch_state_f32(k, io, N, nseq, s, &shape); break;
        case SSU_F16: e = ssu::launch_state_f16(k, io, N, nseq, s, &shape); break;
        default: e = ssu::launch_state_bf16(k, io, N, nseq, s, &shape); break;
    }
    if (log_enabled())
        std::fprintf(stderr,
                     "[ssu] %s: state=%s io=%s dstate=%d heads_per_block=%d loads_per_lane=%d "
                     "xcd_order=%d sr=%d rows_per_block=%u grid=%u block=%u lds=%u B -> %s\n",
                     entry, dtype_name(op.state_dtype), dtype_name(io), N, k.heads_per_block,
                     k.loads_per_lane, k.xcd_order, k.rand_seed != nullptr,
                     shape.rows_per_block, shape.grid, shape.block, shape.lds_bytes,
                     hipGetErrorString(e));
    if (e == hipErrorInvalidConfiguration)
        return fail(SSU_ERR_UNSUPPORTED, "%s: the launch needs more than 2^31-1 workgroups", entry);
    if (e != hipSuccess)
        return fail(SSU_ERR_LAUNCH, "%s: launch failed: %s", entry, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int ssu_one_token(const ssu_one_token_args* a, void* stream) {
    if (!a) return fail(SSU_ERR_INVALID_ARGUMENT, "args must not be NULL");
    if (a->struct_size != sizeof(ssu_one_token_args))
        return fail(SSU_ERR_INVALID_ARGUMENT,
                    "struct_size %u != sizeof(ssu_one_token_args) %zu (header mismatch)",
                    a->struct_size, sizeof(ssu_one_token_args));
    if (a->batch < 0) return fail(SSU_ERR_INVALID_ARGUMENT, "batch must be >= 0");
    if (a->src_slots && !is_index(a->src_dtype))
        return fail(SSU_ERR_INVALID_ARGUMENT, "src_dtype %d is not an ssu_index_dtype", a->src_dtype);
    if (a->dst_slots && !is_index(a->dst_dtype))
        return fail(SSU_ERR_INVALID_ARGUMENT, "dst_dtype %d is not an ssu_index_dtype", a->dst_dtype);
    const ssu_operands& op = a->op;
    if (int rc = check_operands(op, a->batch, a->batch > 0, false)) return rc;
    if (a->batch == 0) return ok();

    ssu::KernelParams k{};
    fill_common(k, op, false, true);
    k.src = a->src_slots;
    k.dst = a->dst_slots;
    k.src_i64 = a->src_dtype == SSU_I64;
    k.dst_i64 = a->dst_dtype == SSU_I64;
    k.rows = a->batch;
    k.packed = 0;
    k.steps = 1;
    return launch(k, op, a->batch, stream, "ssu_one_token");
}

int ssu_packed_varlen(const ssu_packed_args* a, void* stream) {
    if (!a) return fail(SSU_ERR_INVALID_ARGUMENT, "args must not be NULL");
    if (a->struct_size != sizeof(ssu_packed_args))
        return fail(SSU_ERR_INVALID_ARGUMENT,
                    "struct_size %u != sizeof(ssu_packed_args) %zu (header mismatch)",
                    a->struct_size, sizeof(ssu_packed_args));
    if (a->rows < 0 || a->nseq < 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "rows and nseq must be >= 0");
    if (a->seq_len < 0) return fail(SSU_ERR_INVALID_ARGUMENT, "seq_len must be >= 0");
    if (a->cu_seqlens && a->seq_len)
        return fail(SSU_ERR_INVALID_ARGUMENT, "pass either cu_seqlens or seq_len, not both");
    if (a->nseq > 0 && !a->cu_seqlens && !a->seq_len)
        return fail(SSU_ERR_INVALID_ARGUMENT,
                    "cu_seqlens must not be NULL when nseq > 0 (or give seq_len)");
    if ((a->cu_seqlens || a->num_accepted) && !is_index(a->meta_dtype))
        return fail(SSU_ERR_INVALID_ARGUMENT, "meta_dtype %d is not an ssu_index_dtype", a->meta_dtype);
    if (a->num_accepted && !a->src_table)
        return fail(SSU_ERR_INVALID_ARGUMENT,
                    "num_accepted selects an entry of the read table, so src_table is required");
    if (a->src_table && !is_index(a->src_dtype))
        return fail(SSU_ERR_INVALID_ARGUMENT, "src_dtype %d is not an ssu_index_dtype", a->src_dtype);
    if (a->dst_table && !is_index(a->dst_dtype))
        return fail(SSU_ERR_INVALID_ARGUMENT, "dst_dtype %d is not an ssu_index_dtype", a->dst_dtype);
    if ((a->src_table || a->dst_table) && a->steps < 1)
        return fail(SSU_ERR_INVALID_ARGUMENT, "steps must be >= 1 when a slot table is given");
    if (a->src_seq_stride < 0 || a->src_step_stride < 0 || a->dst_seq_stride < 0 ||
        a->dst_step_stride < 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "table strides must be >= 0");
    const ssu_operands& op = a->op;
    const bool work = a->nseq > 0 && a->rows > 0;
    if (int rc = check_operands(op, a->rows, work, true)) return rc;
    if (!work) return ok();
    if (!a->cu_seqlens && a->nseq * a->seq_len != a->rows)
        return fail(SSU_ERR_INVALID_ARGUMENT, "rows (%lld) must equal nseq * seq_len (%lld * %lld)",
                    (long long)a->rows, (long long)a->nseq, (long long)a->seq_len);

    ssu::KernelParams k{};
    fill_common(k, op, true, a->cu_seqlens == nullptr);
    k.src = a->src_table;
    k.dst = a->dst_table;
    k.cu = a->cu_seqlens;
    k.seq_len = a->seq_len;
    k.na = a->num_accepted;
    k.src_seq_stride = a->src_seq_stride;
    k.src_step_stride = a->src_step_stride;
    k.dst_seq_stride = a->dst_seq_stride;
    k.dst_step_stride = a->dst_step_stride;
    k.steps = (a->src_table || a->dst_table) ? a->steps : 1;
    k.src_i64 = a->src_dtype == SSU_I64;
    k.dst_i64 = a->dst_dtype == SSU_I64;
    k.meta_i64 = a->meta_dtype == SSU_I64;
    k.rows = a->rows;
    k.packed = 1;
    return launch(k, op, a->nseq, stream, "ssu_packed_varlen");
}

const char* ssu_last_error(void) { return t_error; }

int ssu_version(void) { return SSU_ABI_VERSION; }

}  // extern "C"
