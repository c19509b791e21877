// C ABI of epx (declared in include/epx.h): host-side validation, sizing and
// kernel launches.  No call allocates, frees or synchronizes; every kernel
// goes onto the caller's stream.
#include <string.h>

#include <mutex>

#include <algorithm>

#include "epx_device.h"

// Built-in workspace of ep_dispatch_layout_noalloc, for callers that cannot
// allocate: zero when the code object loads, and each GPU the library runs
// on holds its own copy for the life of the process.  On the host the name
// is only a stand-in for the device array; host code uses the address
// scratch_address() looks up, never the name.
static __device__ __align__(256) uint8_t scratch[EP_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace epx;

struct Shape {
    int32_t T, H, E, S, K, Kp, A, C, shared, src, E_loc, G, NG;
    int64_t R, min_rows, ws_bytes, tiles, chunks, sp_tiles;
    uint32_t flags;
};

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// A buffer of `bytes` bytes must be present and aligned unless it is empty.
bool bad_buffer(const void* p, int64_t bytes, uintptr_t align) {
    if (bytes == 0) return false;
    return p == nullptr || misaligned(p, align);
}

// Validate `c` and derive the sizes every call needs.
int derive(const ep_cfg_t* c, Shape* d) {
    if (c == nullptr) return EP_EINVAL;
    if (c->num_tokens < 0 || c->hidden < 8 || c->hidden % 8 != 0) return EP_EINVAL;
    if (c->num_experts < 1 || c->num_segments < 1 || c->num_experts % c->num_segments != 0) return EP_EINVAL;
    if (c->top_k < 1 || c->top_k > c->num_experts) return EP_EINVAL;
    if (c->align < 1 || c->align > (1 << 30) || c->seg_capacity < 0) return EP_EINVAL;
    if (c->shared_expert != 0 && c->shared_expert != 1) return EP_EINVAL;
    if (c->shared_expert && (c->src_segment < 0 || c->src_segment >= c->num_segments)) return EP_EINVAL;
    if (c->reserved0 != 0 || c->reserved1 != 0) return EP_EINVAL;
    constexpr uint32_t kPaths = EP_LAYOUT_LOOKBACK | EP_LAYOUT_DIRECT | EP_LAYOUT_BARRIER | EP_LAYOUT_COUNT;
    if (c->flags & ~(EP_ZERO_PAD_ROWS | kPaths)) return EP_EINVAL;
    if (__builtin_popcount(c->flags & kPaths) > 1) return EP_EINVAL;  // at most one path
    if ((c->flags & EP_LAYOUT_COUNT) && (int64_t)c->num_tokens * c->top_k > kCountForcedMaxSlots) return EP_EINVAL;
    if ((c->flags & EP_LAYOUT_BARRIER) && (int64_t)c->num_tokens * c->top_k > kBarrierForcedMaxSlots) return EP_EINVAL;
    d->T = c->num_tokens;
    d->H = c->hidden;
    d->E = c->num_experts;
    d->S = c->num_segments;
    d->K = c->top_k;
    d->shared = c->shared_expert;
    d->Kp = d->K + d->shared;
    if (d->Kp > kMaxSlots) return EP_EINVAL;  // a token's slots are spread over one wave's lanes
    d->A = c->align;
    d->C = c->seg_capacity;
    d->src = d->shared ? c->src_segment : 0;
    d->E_loc = d->E / d->S;
    d->G = d->E_loc + d->shared;
    const int64_t ng = (int64_t)d->S * d->G;
    if (ng > EP_MAX_GROUPS) return EP_EINVAL;
    d->NG = (int32_t)ng;
    const int64_t slots = (int64_t)d->T * d->Kp;
    if (slots >= (int64_t(1) << 30)) return EP_EINVAL;  // look-back descriptors hold 30-bit counts
    // Every group is padded by at most A - 1 rows, so the used rows of all
    // segments before any capacity clamp are at most `packed`.  The layout
    // kernels add up the aligned group sizes in int32 before clamping them to
    // C, so this bound must fit in int32 in capacity mode too.
    const int64_t groups = (int64_t)d->E + d->shared;
    const int64_t packed = slots + (slots < groups ? slots : groups) * (int64_t)(d->A - 1);
    if (packed >= (int64_t(1) << 31)) return EP_EINVAL;
    d->min_rows = d->C > 0 ? (int64_t)d->S * d->C : packed;
    if (d->min_rows >= (int64_t(1) << 31)) return EP_EINVAL;  // rows are int32
    // Workspace: a header, then either path's tables (the direct path's
    // 32-bit tile counts and chunk sums; the single pass's two arrays of
    // 64-bit descriptors).
    d->tiles = layout_tiles((int64_t)d->T * d->K, d->NG);
    d->chunks = direct_chunks(d->tiles);
    d->sp_tiles = sp_tiles((int64_t)d->T * d->K);
    d->ws_bytes = kWorkspaceHeader + std::max((d->tiles + d->chunks) * (int64_t)d->NG * 4,
                                              d->sp_tiles * (int64_t)d->NG * 16);
    d->R = c->recv_rows;
    d->flags = c->flags;
    return EP_OK;
}

int check_rows(const Shape& d) {
    if (d.R < d.min_rows || d.R >= (int64_t(1) << 31)) return EP_EINVAL;
    return EP_OK;
}

// The current device must be a gfx950; the answer is cached per device.
int check_device() {
    static std::mutex mu;
    static int arch_state[64];  // 0 unknown, 1 ok, 2 not supported
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return EP_ELAUNCH;
    if (dev < 0 || dev >= 64) return EP_ENOTSUP;
    std::lock_guard<std::mutex> lock(mu);
    if (arch_state[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return EP_ELAUNCH;
        arch_state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return arch_state[dev] == 1 ? EP_OK : EP_ENOTSUP;
}

int status_of(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ELAUNCH; }

// Kernels that launch one grid for the whole batch, with `per_token`
// work-items per token: a grid dimension holds at most 2^32 - 1 work-items
// (the movers split larger batches into chunks instead).
bool grid_too_big(const Shape& d, int64_t per_token) {
    return (int64_t)d.T * per_token + 1024 > 0xFFFFFFFFll;
}

// Layout arrays read by the payload calls.
int check_layout_for_payload(const Shape& d, const ep_layout_t* L) {
    if (L == nullptr) return EP_EINVAL;
    if (bad_buffer(L->token_row, (int64_t)d.T * d.Kp * 4, 4)) return EP_EINVAL;
    if (d.flags & EP_ZERO_PAD_ROWS) {
        if (bad_buffer(L->counts, (int64_t)d.NG * 4, 4) ||
            bad_buffer(L->row_offsets, (int64_t)d.S * (d.G + 1) * 4, 4) ||
            bad_buffer(L->seg_base, (int64_t)(d.S + 1) * 4, 4))
            return EP_EINVAL;
    }
    return EP_OK;
}

MoveArgs move_args(const Shape& d, const ep_layout_t* L, const void* src, void* dst, const float* probs) {
    MoveArgs m;
    m.src = src;
    m.dst = dst;
    m.token_row = L->token_row;
    m.probs = probs;
    m.T = d.T;
    m.K = d.K;
    m.Kp = d.Kp;
    m.H = d.H;
    m.R = d.R;
    return m;
}

int zero_pad(const Shape& d, const ep_layout_t* L, void* base, int64_t row_bytes, hipStream_t st) {
    if (!(d.flags & EP_ZERO_PAD_ROWS) || d.A == 1) return EP_OK;
    return status_of(launch_zero_pad_rows(base, row_bytes, *L, d.S, d.G, d.A, d.C, d.R, st));
}

Nvfp4Args nvfp4_args(const Shape& d, const ep_layout_t* L, const uint16_t* x, uint8_t* codes, uint8_t* scales,
                     uint16_t* rowscale) {
    Nvfp4Args a;
    a.x = x;
    a.codes = codes;
    a.scales = scales;
    a.rowscale = rowscale;
    a.token_row = L->token_row;
    a.T = d.T;
    a.Kp = d.Kp;
    a.H = d.H;
    a.R = d.R;
    return a;
}

Fp8Args fp8_args(const Shape& d, const ep_layout_t* L, const uint16_t* x, uint8_t* codes, float* scales) {
    Fp8Args a;
    a.x = x;
    a.codes = codes;
    a.scales = scales;
    a.token_row = L->token_row;
    a.T = d.T;
    a.Kp = d.Kp;
    a.H = d.H;
    a.R = d.R;
    return a;
}

int zero_pad_fp8(const Shape& d, const ep_layout_t* L, uint8_t* codes, float* scales, hipStream_t st) {
    int rc;
    if ((rc = zero_pad(d, L, codes, d.H, st)) != EP_OK) return rc;
    return zero_pad(d, L, scales, (int64_t)(d.H / 128) * 4, st);
}

int zero_pad_nvfp4(const Shape& d, const ep_layout_t* L, uint8_t* codes, uint8_t* scales, uint16_t* rowscale,
                   hipStream_t st) {
    int rc;
    if ((rc = zero_pad(d, L, codes, d.H / 2, st)) != EP_OK) return rc;
    if ((rc = zero_pad(d, L, scales, d.H / 16, st)) != EP_OK) return rc;
    return zero_pad(d, L, rowscale, 2, st);
}

// Host-side checks shared by both layout entry points (everything but the
// workspace).
int layout_check(const Shape& d, const int32_t* topk_ids, const ep_layout_t* L) {
    int rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if ((int64_t)d.T * d.K > kLayoutMaxSlots) return EP_EINVAL;
    if (L == nullptr) return EP_EINVAL;
    if (bad_buffer(topk_ids, (int64_t)d.T * d.K * 4, 4)) return EP_EINVAL;
    if (bad_buffer(L->counts, (int64_t)d.NG * 4, 4) || bad_buffer(L->seg_base, (int64_t)(d.S + 1) * 4, 4) ||
        bad_buffer(L->row_offsets, (int64_t)d.S * (d.G + 1) * 4, 4) ||
        bad_buffer(L->scales_offsets, (int64_t)d.S * (d.G + 1) * 4, 4) ||
        bad_buffer(L->token_row, (int64_t)d.T * d.Kp * 4, 4) || bad_buffer(L->expert_ids, d.R * 4, 4) ||
        bad_buffer(L->src_info, d.R * 8, 8) || bad_buffer(L->flags, 4, 4))
        return EP_EINVAL;
    return EP_OK;
}

// Launch of the layout kernels, after layout_check and check_device; `ws`
// holds at least d.ws_bytes bytes.  With x and one dispatch's outputs given
// (out), the small path also makes that bf16, NVFP4 or FP8 dispatch
// (*fused is set when it did).
struct FusedOut {  // the dispatch a small-path layout launch makes beside the layout
    uint16_t* recv = nullptr;
    uint8_t* codes = nullptr;
    uint8_t* scales = nullptr;
    uint16_t* rowscale = nullptr;
    uint8_t* f8_codes = nullptr;
    float* f8_scales = nullptr;
};

int layout_launch(const Shape& d, const int32_t* topk_ids, void* ws, const ep_layout_t* L, void* stream,
                  const uint16_t* x = nullptr, const FusedOut& out = FusedOut(), bool* fused = nullptr) {
    LayoutArgs a;
    a.x = nullptr;
    a.recv = nullptr;
    a.codes = nullptr;
    a.scales = nullptr;
    a.rowscale = nullptr;
    a.f8_codes = nullptr;
    a.f8_scales = nullptr;
    a.fused_rpu = 1;
    a.H = d.H;
    a.topk_ids = topk_ids;
    a.desc = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + kWorkspaceHeader);
    a.out = *L;
    a.T = d.T;
    a.K = d.K;
    a.Kp = d.Kp;
    a.E = d.E;
    a.S = d.S;
    a.G = d.G;
    a.NG = d.NG;
    a.E_loc = d.E_loc;
    a.A = d.A;
    a.C = d.C;
    a.shared = d.shared;
    a.src_seg = d.src;
    a.recv_rows = d.R;
    a.sp_header = ws;
    a.sp_desc = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + kWorkspaceHeader);
    const int64_t routed = (int64_t)d.T * d.K;
    a.lookback = 0;
    if (d.flags & EP_LAYOUT_LOOKBACK) {
        a.mode = kLayoutSinglePass;
        a.lookback = 1;
    } else if (d.flags & EP_LAYOUT_BARRIER) {
        a.mode = kLayoutSinglePass;
    } else if (d.flags & EP_LAYOUT_DIRECT) {
        a.mode = kLayoutDirect;
    } else if (d.flags & EP_LAYOUT_COUNT) {
        a.mode = kLayoutCount;
    } else if (routed <= kSmallMaxSlots) {
        a.mode = kLayoutSmall;
    } else if (routed <= kCountMaxSlots) {
        a.mode = kLayoutCount;
    } else {
        a.mode = kLayoutDirect;  // measured faster than the single pass at every size
    }
    a.chunks = 0;
    a.chunk_sums = nullptr;
    if (a.mode == kLayoutSinglePass) {
        a.tiles = (int32_t)d.sp_tiles;
        a.rank_blocks = (int32_t)sp_blocks(d.sp_tiles, d.NG);
        a.slots_per_thread = sp_slots_per_thread(routed);
    } else if (a.mode == kLayoutCount) {
        a.slots_per_thread = 1;
        a.tiles = (int32_t)std::max<int64_t>(1, (routed + kLayoutThreads - 1) / kLayoutThreads);
        a.rank_blocks = (int32_t)std::max<int64_t>(a.tiles, std::min<int32_t>(d.NG, 256));
    } else if (a.mode == kLayoutDirect) {
        a.tiles = (int32_t)d.tiles;
        a.chunks = (int32_t)d.chunks;
        if (d.chunks > 0) a.chunk_sums = a.desc + d.tiles * (int64_t)d.NG;
        a.rank_blocks = (int32_t)std::max<int64_t>(d.tiles, std::min<int32_t>(d.NG, 256));
        a.slots_per_thread = layout_slots_per_thread(routed, d.NG);
    } else {  // one tile holds every slot
        a.tiles = 1;
        a.rank_blocks = std::min<int32_t>(d.NG, 256);
        a.slots_per_thread = routed <= 256 ? 1 : (routed <= 512 ? 2 : 4);
        a.x = x;
        a.recv = out.recv;
        a.codes = out.codes;
        a.scales = out.scales;
        a.rowscale = out.rowscale;
        a.f8_codes = out.f8_codes;
        a.f8_scales = out.f8_scales;
        if (x != nullptr) {
            // A fused dispatch unit is a token and up to rpu of its K' rows:
            // the fewest rows per unit whose units fit one round of
            // workgroups, so that as many tokens as possible are read (and
            // quantized) once per unit and no workgroup takes two units.
            // Measured at DeepSeek-V3 dims, T = 40 and 64: NVFP4 7.8 and 7.9
            // us against 9.0 and 9.1 with one token (all rows) per unit.
            const int64_t items = (int64_t)d.T * d.Kp, grid = a.rank_blocks;
            int32_t r = (int32_t)std::min<int64_t>(d.Kp, std::max<int64_t>(1, (items + grid - 1) / grid));
            while (r < d.Kp && (int64_t)d.T * ((d.Kp + r - 1) / r) > grid) ++r;
            a.fused_rpu = r;
        }
    }
    if (fused) *fused = a.x != nullptr;
    return status_of(launch_layout(a, static_cast<hipStream_t>(stream)));
}

constexpr int64_t kScratchBytes = EP_NOALLOC_SCRATCH_BYTES;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return EP_ELAUNCH;
    if (dev < 0 || dev >= 64) return EP_ENOTSUP;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return EP_ELAUNCH;
        addr[dev] = p;
    }
    *out = addr[dev];
    return EP_OK;
}

}  // namespace

extern "C" {

int ep_abi_version(void) { return EPX_ABI_VERSION; }

const char* ep_strerror(int status) {
    switch (status) {
        case EP_OK: return "ok";
        case EP_EINVAL: return "invalid argument";
        case EP_ELAUNCH: return "HIP runtime error while enqueueing work";
        case EP_ENOTSUP: return "device is not gfx950 (MI355X)";
        case EP_ESCRATCH:
            return "the layout needs more scratch than the built-in buffer of ep_dispatch_layout_noalloc "
                   "holds (EP_NOALLOC_SCRATCH_BYTES); use ep_dispatch_layout with a workspace";
        default: return "unknown status";
    }
}

int ep_query(const ep_cfg_t* cfg, int64_t* min_recv_rows, int64_t* workspace_bytes, int32_t* groups_per_seg) {
    Shape d;
    const int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if (min_recv_rows) *min_recv_rows = d.min_rows;
    if (workspace_bytes) *workspace_bytes = d.ws_bytes;
    if (groups_per_seg) *groups_per_seg = d.G;
    return EP_OK;
}

int ep_dispatch_layout(const ep_cfg_t* cfg, const int32_t* topk_ids, void* workspace, int64_t workspace_bytes,
                       const ep_layout_t* layout, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = layout_check(d, topk_ids, layout)) != EP_OK) return rc;
    if (workspace == nullptr || misaligned(workspace, 16) || workspace_bytes < d.ws_bytes) return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    return layout_launch(d, topk_ids, workspace, layout, stream);
}

int ep_dispatch_layout_noalloc(const ep_cfg_t* cfg, const int32_t* topk_ids, const ep_layout_t* layout,
                               void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = layout_check(d, topk_ids, layout)) != EP_OK) return rc;
    if (d.ws_bytes > kScratchBytes) return EP_ESCRATCH;
    if ((rc = check_device()) != EP_OK) return rc;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws)) != EP_OK) return rc;
    return layout_launch(d, topk_ids, ws, layout, stream);
}

int ep_dispatch(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* x, uint16_t* recv, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if ((rc = check_layout_for_payload(d, layout)) != EP_OK) return rc;
    if (bad_buffer(x, (int64_t)d.T * d.H * 2, 16) || bad_buffer(recv, d.R * d.H * 2, 16)) return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = status_of(launch_scatter(move_args(d, layout, x, recv, nullptr), st))) != EP_OK) return rc;
    return zero_pad(d, layout, recv, (int64_t)d.H * 2, st);
}

int ep_dispatch_with_layout(const ep_cfg_t* cfg, const int32_t* topk_ids, void* workspace, int64_t workspace_bytes,
                            const ep_layout_t* layout, const uint16_t* x, uint16_t* recv, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = layout_check(d, topk_ids, layout)) != EP_OK) return rc;
    if (workspace == nullptr || misaligned(workspace, 16) || workspace_bytes < d.ws_bytes) return EP_EINVAL;
    if (bad_buffer(x, (int64_t)d.T * d.H * 2, 16) || bad_buffer(recv, d.R * d.H * 2, 16)) return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool fused = false;
    FusedOut out;
    out.recv = recv;
    if ((rc = layout_launch(d, topk_ids, workspace, layout, stream, x, out, &fused)) != EP_OK) return rc;
    if (!fused && (rc = status_of(launch_scatter(move_args(d, layout, x, recv, nullptr), st))) != EP_OK) return rc;
    return zero_pad(d, layout, recv, (int64_t)d.H * 2, st);
}

int ep_dispatch_nvfp4(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* x, uint8_t* codes,
                      uint8_t* scales, uint16_t* rowscale, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if (d.H % 16 != 0 || d.H > nvfp4_max_hidden() || grid_too_big(d, 64)) return EP_EINVAL;
    if ((rc = check_layout_for_payload(d, layout)) != EP_OK) return rc;
    if (bad_buffer(x, (int64_t)d.T * d.H * 2, 16) || bad_buffer(codes, d.R * (d.H / 2), 16) ||
        bad_buffer(scales, d.R * (d.H / 16), 1) || bad_buffer(rowscale, d.R * 2, 2))
        return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = status_of(launch_nvfp4(nvfp4_args(d, layout, x, codes, scales, rowscale), st))) != EP_OK) return rc;
    return zero_pad_nvfp4(d, layout, codes, scales, rowscale, st);
}

int ep_dispatch_nvfp4_with_layout(const ep_cfg_t* cfg, const int32_t* topk_ids, void* workspace,
                                  int64_t workspace_bytes, const ep_layout_t* layout, const uint16_t* x,
                                  uint8_t* codes, uint8_t* scales, uint16_t* rowscale, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = layout_check(d, topk_ids, layout)) != EP_OK) return rc;
    if (workspace == nullptr || misaligned(workspace, 16) || workspace_bytes < d.ws_bytes) return EP_EINVAL;
    if (d.H % 16 != 0 || d.H > nvfp4_max_hidden() || grid_too_big(d, 64)) return EP_EINVAL;
    if (bad_buffer(x, (int64_t)d.T * d.H * 2, 16) || bad_buffer(codes, d.R * (d.H / 2), 16) ||
        bad_buffer(scales, d.R * (d.H / 16), 1) || bad_buffer(rowscale, d.R * 2, 2))
        return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool fused = false;
    FusedOut out;
    out.codes = codes;
    out.scales = scales;
    out.rowscale = rowscale;
    if ((rc = layout_launch(d, topk_ids, workspace, layout, stream, x, out, &fused)) != EP_OK) return rc;
    if (!fused && (rc = status_of(launch_nvfp4(nvfp4_args(d, layout, x, codes, scales, rowscale), st))) != EP_OK)
        return rc;
    return zero_pad_nvfp4(d, layout, codes, scales, rowscale, st);
}

int ep_dispatch_fp8(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* x, uint8_t* codes,
                    float* scales, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if (d.H % 128 != 0 || d.H > fp8_max_hidden() || grid_too_big(d, 64)) return EP_EINVAL;
    if ((rc = check_layout_for_payload(d, layout)) != EP_OK) return rc;
    if (bad_buffer(x, (int64_t)d.T * d.H * 2, 16) || bad_buffer(codes, d.R * d.H, 16) ||
        bad_buffer(scales, d.R * (d.H / 128) * 4, 4))
        return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = status_of(launch_fp8(fp8_args(d, layout, x, codes, scales), st))) != EP_OK) return rc;
    return zero_pad_fp8(d, layout, codes, scales, st);
}

int ep_dispatch_fp8_with_layout(const ep_cfg_t* cfg, const int32_t* topk_ids, void* workspace,
                                int64_t workspace_bytes, const ep_layout_t* layout, const uint16_t* x,
                                uint8_t* codes, float* scales, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = layout_check(d, topk_ids, layout)) != EP_OK) return rc;
    if (workspace == nullptr || misaligned(workspace, 16) || workspace_bytes < d.ws_bytes) return EP_EINVAL;
    if (d.H % 128 != 0 || d.H > fp8_max_hidden() || grid_too_big(d, 64)) return EP_EINVAL;
    if (bad_buffer(x, (int64_t)d.T * d.H * 2, 16) || bad_buffer(codes, d.R * d.H, 16) ||
        bad_buffer(scales, d.R * (d.H / 128) * 4, 4))
        return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool fused = false;
    FusedOut out;
    out.f8_codes = codes;
    out.f8_scales = scales;
    if ((rc = layout_launch(d, topk_ids, workspace, layout, stream, x, out, &fused)) != EP_OK) return rc;
    if (!fused && (rc = status_of(launch_fp8(fp8_args(d, layout, x, codes, scales), st))) != EP_OK) return rc;
    return zero_pad_fp8(d, layout, codes, scales, st);
}

int ep_combine(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* expert_out, const float* probs,
               uint16_t* y, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if (layout == nullptr || bad_buffer(layout->token_row, (int64_t)d.T * d.Kp * 4, 4)) return EP_EINVAL;
    if (bad_buffer(expert_out, d.R * d.H * 2, 16) || bad_buffer(y, (int64_t)d.T * d.H * 2, 16)) return EP_EINVAL;
    if (probs != nullptr && misaligned(probs, 4)) return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    return status_of(launch_gather_reduce(move_args(d, layout, expert_out, y, probs), static_cast<hipStream_t>(stream)));
}

int ep_combine_nvfp4(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint8_t* codes, const uint8_t* scales,
                     const uint16_t* rowscale, const float* probs, uint16_t* y, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if (d.H % 16 != 0 || grid_too_big(d, (int64_t)kWave * combine_nvfp4_pieces(d.H))) return EP_EINVAL;
    if (layout == nullptr || bad_buffer(layout->token_row, (int64_t)d.T * d.Kp * 4, 4)) return EP_EINVAL;
    if (bad_buffer(codes, d.R * (d.H / 2), 8) || bad_buffer(scales, d.R * (d.H / 16), 1) ||
        bad_buffer(rowscale, d.R * 2, 2) || bad_buffer(y, (int64_t)d.T * d.H * 2, 16))
        return EP_EINVAL;
    if (probs != nullptr && misaligned(probs, 4)) return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    CombineNvfp4Args a;
    a.codes = codes;
    a.scales = scales;
    a.rowscale = rowscale;
    a.token_row = layout->token_row;
    a.probs = probs;
    a.y = y;
    a.T = d.T;
    a.K = d.K;
    a.Kp = d.Kp;
    a.H = d.H;
    a.R = d.R;
    return status_of(launch_combine_nvfp4(a, static_cast<hipStream_t>(stream)));
}

int ep_dispatch_bwd(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* grad_recv, uint16_t* grad_x,
                    void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if (layout == nullptr || bad_buffer(layout->token_row, (int64_t)d.T * d.Kp * 4, 4)) return EP_EINVAL;
    if (bad_buffer(grad_recv, d.R * d.H * 2, 16) || bad_buffer(grad_x, (int64_t)d.T * d.H * 2, 16)) return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    return status_of(launch_gather_reduce(move_args(d, layout, grad_recv, grad_x, nullptr), static_cast<hipStream_t>(stream)));
}

int ep_combine_bwd(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* grad_y, const float* probs,
                   uint16_t* grad_expert_out, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if ((rc = check_layout_for_payload(d, layout)) != EP_OK) return rc;
    if (bad_buffer(grad_y, (int64_t)d.T * d.H * 2, 16) || bad_buffer(grad_expert_out, d.R * d.H * 2, 16))
        return EP_EINVAL;
    if (probs != nullptr && misaligned(probs, 4)) return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const MoveArgs m = move_args(d, layout, grad_y, grad_expert_out, probs);
    rc = status_of(probs != nullptr ? launch_scatter_scaled(m, st) : launch_scatter(m, st));
    if (rc != EP_OK) return rc;
    return zero_pad(d, layout, grad_expert_out, (int64_t)d.H * 2, st);
}

int ep_combine_bwd_probs(const ep_cfg_t* cfg, const ep_layout_t* layout, const uint16_t* grad_y,
                         const uint16_t* expert_out, float* grad_probs, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if ((rc = check_rows(d)) != EP_OK) return rc;
    if (layout == nullptr || bad_buffer(layout->token_row, (int64_t)d.T * d.Kp * 4, 4)) return EP_EINVAL;
    if (grid_too_big(d, 256)) return EP_EINVAL;
    if (bad_buffer(grad_y, (int64_t)d.T * d.H * 2, 16) || bad_buffer(expert_out, d.R * d.H * 2, 16) ||
        bad_buffer(grad_probs, (int64_t)d.T * d.K * 4, 4))
        return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    MoveArgs m = move_args(d, layout, grad_y, const_cast<uint16_t*>(expert_out), nullptr);
    return status_of(launch_probs_grad(m, grad_probs, static_cast<hipStream_t>(stream)));
}

int ep_indices_to_multihot(const ep_cfg_t* cfg, const int32_t* topk_ids, const float* probs,
                           uint8_t* routing_map, float* dense_probs, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if (grid_too_big(d, 64)) return EP_EINVAL;
    if (bad_buffer(topk_ids, (int64_t)d.T * d.K * 4, 4) || bad_buffer(routing_map, (int64_t)d.T * d.E, 1))
        return EP_EINVAL;
    if (dense_probs != nullptr && (bad_buffer(dense_probs, (int64_t)d.T * d.E * 4, 4) ||
                                   bad_buffer(probs, (int64_t)d.T * d.K * 4, 4)))
        return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    RouteArgs a;
    a.ids = const_cast<int32_t*>(topk_ids);
    a.probs = dense_probs != nullptr ? const_cast<float*>(probs) : nullptr;
    a.map = routing_map;
    a.dense_probs = dense_probs;
    a.flags = nullptr;
    a.T = d.T;
    a.K = d.K;
    a.E = d.E;
    return status_of(launch_indices_to_multihot(a, static_cast<hipStream_t>(stream)));
}

int ep_multihot_to_indices(const ep_cfg_t* cfg, const uint8_t* routing_map, const float* dense_probs,
                           int32_t* topk_ids, float* probs, int32_t* flags, void* stream) {
    Shape d;
    int rc = derive(cfg, &d);
    if (rc != EP_OK) return rc;
    if (grid_too_big(d, 64)) return EP_EINVAL;
    if (bad_buffer(routing_map, (int64_t)d.T * d.E, 1) || bad_buffer(topk_ids, (int64_t)d.T * d.K * 4, 4))
        return EP_EINVAL;
    if (probs != nullptr && (bad_buffer(probs, (int64_t)d.T * d.K * 4, 4) ||
                             bad_buffer(dense_probs, (int64_t)d.T * d.E * 4, 4)))
        return EP_EINVAL;
    if (flags != nullptr && misaligned(flags, 4)) return EP_EINVAL;
    if ((rc = check_device()) != EP_OK) return rc;
    RouteArgs a;
    a.ids = topk_ids;
    a.probs = probs;
    a.map = const_cast<uint8_t*>(routing_map);
    a.dense_probs = probs != nullptr ? const_cast<float*>(dense_probs) : nullptr;
    a.flags = flags;
    a.T = d.T;
    a.K = d.K;
    a.E = d.E;
    return status_of(launch_multihot_to_indices(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
