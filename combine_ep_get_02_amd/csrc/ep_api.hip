// ep_api.hip -- the extern "C" entry points of libep.so (declared in ep.h):
// argument checks, then kernel launches on the caller's stream.
//
// Every check runs on the host before anything is enqueued, so a rejected call
// leaves the stream untouched.  The argument rules restate the host asserts of
// the mscclpp ht_runtime.cc mirror (constructor: fewer than 8 ranks or a
// multiple of 8; experts split evenly over ranks; rows a whole number of
// 16-byte units in internodeCombine / intranodeCombine).
#include <limits.h>

#include "ep_internal.h"

namespace {

using namespace ep;

ep_status_t check_shape(const ep_shape_t *s) {
    if (s == nullptr) return EP_ERR_INVALID_ARG;
    if (s->num_tokens < 0 || s->hidden < 8 || s->hidden % 8 != 0 || s->num_topk < 1 || s->num_experts < 1 ||
        s->num_ranks < 1 || s->num_channels < 1 || s->expert_alignment < 1 || s->my_rank < 0 ||
        s->my_rank >= s->num_ranks)
        return EP_ERR_INVALID_ARG;
    if (s->num_ranks >= kRanksPerNode && s->num_ranks % kRanksPerNode != 0) return EP_ERR_INVALID_ARG;
    if (s->num_experts % s->num_ranks != 0) return EP_ERR_INVALID_ARG;
    if (s->num_ranks > kMaxRanks || s->num_topk > kMaxTopk || s->num_channels > kMaxChannels)
        return EP_ERR_UNSUPPORTED;
    // every receive row index and every send_slot entry must fit int32
    if ((int64_t)s->num_tokens * s->num_ranks > INT_MAX) return EP_ERR_UNSUPPORTED;
    return EP_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool form_ok(int32_t form) { return form == EP_FORM_AUTO || form == EP_FORM_PUSH || form == EP_FORM_PULL; }

ep_status_t from_hip(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

bool workspace_ok(const ep_shape_t *s, const void *ws, size_t bytes) {
    return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0 &&
           bytes >= workspace_layout(s->num_tokens, s->num_ranks, s->num_experts, s->num_channels, s->num_topk).total;
}

// The routing inputs of a dispatch: is_token_in_rank, the channel prefix matrix and
// the receive prefix sums are required; the workspace is optional (NULL: the routing
// is worked out from those inputs, which needs channels of at most
// kMaxDeriveChannelTokens tokens), and when given it must be a whole workspace.
ep_status_t routing_checked(const ep_shape_t *s, const uint8_t *in_rank, const int32_t *gbl,
                            const int32_t *recv_gbl, const void *workspace, size_t workspace_bytes) {
    if (in_rank == nullptr || gbl == nullptr || recv_gbl == nullptr) return EP_ERR_INVALID_ARG;
    if (workspace != nullptr) return workspace_ok(s, workspace, workspace_bytes) ? EP_OK : EP_ERR_INVALID_ARG;
    const int64_t tc = ((int64_t)s->num_tokens + s->num_channels - 1) / s->num_channels;
    return tc <= kMaxDeriveChannelTokens ? EP_OK : EP_ERR_UNSUPPORTED;
}

// Shared checks and launch of the bf16, fp8 and quantising dispatch entry points.
// quant_log2 >= 0: x is bf16, rows leave as E4M3 codes of row_bytes bytes with
// num_scales scales made on the way (x_scales is not read); -1 otherwise.
ep_status_t dispatch_checked(const ep_shape_t *s, const void *x, int64_t row_bytes, const float *x_scales,
                             int32_t num_scales, const int64_t *topk_idx, const float *topk_weights,
                             const uint8_t *is_token_in_rank, const int32_t *gbl_channel_prefix_matrix,
                             const int32_t *recv_gbl_rank_prefix_sum, const void *workspace, size_t workspace_bytes,
                             int32_t recv_capacity, void *recv_x, float *recv_x_scales, float *recv_topk_weights,
                             int64_t *recv_topk_idx, int32_t *recv_src_info, int32_t *send_slot, int32_t form,
                             int32_t *dev_status, hipStream_t stream, int quant_log2 = -1) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (row_bytes % 16 != 0 || recv_capacity < 0 || num_scales < 0 || !form_ok(form)) return EP_ERR_INVALID_ARG;
    if (num_scales > kMaxScales) return EP_ERR_UNSUPPORTED;
    if (s->num_tokens == 0) return EP_OK;
    if (x == nullptr || topk_idx == nullptr || topk_weights == nullptr || send_slot == nullptr)
        return EP_ERR_INVALID_ARG;
    if (recv_capacity > 0 && (recv_x == nullptr || recv_topk_weights == nullptr || recv_src_info == nullptr))
        return EP_ERR_INVALID_ARG;
    if (num_scales > 0 && ((quant_log2 < 0 && x_scales == nullptr) || (recv_capacity > 0 && recv_x_scales == nullptr)))
        return EP_ERR_INVALID_ARG;
    if (!aligned16(x) || (recv_x != nullptr && !aligned16(recv_x))) return EP_ERR_INVALID_ARG;
    if (recv_src_info != nullptr && (reinterpret_cast<uintptr_t>(recv_src_info) & 7u) != 0) return EP_ERR_INVALID_ARG;
    st = routing_checked(s, is_token_in_rank, gbl_channel_prefix_matrix, recv_gbl_rank_prefix_sum, workspace,
                         workspace_bytes);
    if (st != EP_OK) return st;
    DispatchArgs a = {};
    a.x = x;
    a.row_units = row_bytes / 16;
    a.x_scales = x_scales;
    a.num_scales = num_scales;
    a.topk_idx = topk_idx;
    a.topk_w = topk_weights;
    a.in_rank = is_token_in_rank;
    a.gbl = gbl_channel_prefix_matrix;
    a.recv_gbl = recv_gbl_rank_prefix_sum;
    a.ws = static_cast<const char *>(workspace);
    a.cached_slot = nullptr;
    a.cap = recv_capacity;
    a.recv_x = recv_x;
    a.recv_scales = recv_x_scales;
    a.recv_w = recv_topk_weights;
    a.recv_idx = recv_topk_idx;
    a.src_info = recv_src_info;
    a.send_slot = send_slot;
    a.form = form;
    a.dev_status = dev_status;
    a.quantize = quant_log2 >= 0;
    a.quant_log2 = quant_log2 >= 0 ? quant_log2 : 0;
    return from_hip(launch_dispatch(*s, a, stream));
}

// Shared checks of the quantiser and the dequantiser: rows >= 0, hidden a positive multiple of
// 16, groups of 16 << l channels (0 <= l <= 6), rows and code buffers 16-byte aligned, scales
// 4-byte aligned.
ep_status_t quant_checked(const void *rows16, const void *codes, const float *scales, int64_t num_rows,
                          int32_t hidden, int32_t num_scales) {
    if (num_rows < 0 || hidden < kQuantChannels || hidden % kQuantChannels != 0 || num_scales < 1 ||
        hidden % num_scales != 0)
        return EP_ERR_INVALID_ARG;
    if (quant_lanes_log2(hidden, num_scales) < 0) return EP_ERR_UNSUPPORTED;
    if (num_rows == 0) return EP_OK;
    if (rows16 == nullptr || codes == nullptr || scales == nullptr) return EP_ERR_INVALID_ARG;
    if (!aligned16(rows16) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
        return EP_ERR_INVALID_ARG;
    return EP_OK;
}

}  // namespace

extern "C" {

const char *ep_status_string(ep_status_t status) {
    switch (status) {
        case EP_OK: return "EP_OK";
        case EP_ERR_INVALID_ARG: return "EP_ERR_INVALID_ARG: malformed shape or pointer";
        case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED: shape beyond this version's limits";
        case EP_ERR_HIP: return "EP_ERR_HIP: a HIP launch or copy failed";
    }
    return "unknown ep_status_t";
}

size_t ep_workspace_bytes(const ep_shape_t *s) {
    if (check_shape(s) != EP_OK) return 0;
    return workspace_layout(s->num_tokens, s->num_ranks, s->num_experts, s->num_channels, s->num_topk).total;
}

ep_status_t ep_get_layout(const ep_shape_t *s, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                          int32_t *num_tokens_per_rdma_rank, int32_t *num_tokens_per_expert,
                          uint8_t *is_token_in_rank, void *workspace, size_t workspace_bytes, int32_t *dev_status,
                          hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (num_tokens_per_rank == nullptr || num_tokens_per_rdma_rank == nullptr || num_tokens_per_expert == nullptr)
        return EP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && (topk_idx == nullptr || is_token_in_rank == nullptr)) return EP_ERR_INVALID_ARG;
    if (!workspace_ok(s, workspace, workspace_bytes)) return EP_ERR_INVALID_ARG;
    return from_hip(launch_layout(*s, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank,
                                  num_tokens_per_expert, is_token_in_rank, static_cast<char *>(workspace),
                                  dev_status, stream));
}

ep_status_t ep_get_layout_noalloc(const ep_shape_t *s, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                                  int32_t *num_tokens_per_rdma_rank, int32_t *num_tokens_per_expert,
                                  uint8_t *is_token_in_rank, int32_t *dev_status, hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (num_tokens_per_rank == nullptr || num_tokens_per_rdma_rank == nullptr || num_tokens_per_expert == nullptr)
        return EP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && (topk_idx == nullptr || is_token_in_rank == nullptr)) return EP_ERR_INVALID_ARG;
    if (s->num_experts > kNoallocMaxExperts) return EP_ERR_UNSUPPORTED;
    // the stream must belong to the current device, whose scratch the call uses
    int device = -1, stream_device = -1;
    if (hipGetDevice(&device) != hipSuccess || hipStreamGetDevice(stream, &stream_device) != hipSuccess)
        return EP_ERR_HIP;
    if (device != stream_device) return EP_ERR_INVALID_ARG;
    return from_hip(launch_layout_noalloc(*s, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank,
                                          num_tokens_per_expert, is_token_in_rank, dev_status, stream));
}

ep_status_t ep_notify(const ep_shape_t *s, const uint8_t *is_token_in_rank, const int32_t *num_tokens_per_rank,
                      const int32_t *num_tokens_per_rdma_rank, const int32_t *num_tokens_per_expert,
                      int32_t *gbl_channel_prefix_matrix, int32_t *rdma_channel_prefix_matrix,
                      int32_t *recv_gbl_rank_prefix_sum, int32_t *recv_rdma_rank_prefix_sum,
                      int32_t *num_recv_tokens_per_expert, int32_t *num_recv_tokens, int32_t *num_recv_tokens_host,
                      void *workspace, size_t workspace_bytes, int32_t *dev_status, hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (num_tokens_per_rank == nullptr || num_tokens_per_rdma_rank == nullptr || num_tokens_per_expert == nullptr ||
        gbl_channel_prefix_matrix == nullptr || rdma_channel_prefix_matrix == nullptr ||
        recv_gbl_rank_prefix_sum == nullptr || recv_rdma_rank_prefix_sum == nullptr ||
        num_recv_tokens_per_expert == nullptr || num_recv_tokens == nullptr)
        return EP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && is_token_in_rank == nullptr) return EP_ERR_INVALID_ARG;
    if (!workspace_ok(s, workspace, workspace_bytes)) return EP_ERR_INVALID_ARG;
    hipError_t e = launch_notify(*s, is_token_in_rank, num_tokens_per_rank, num_tokens_per_rdma_rank,
                                 num_tokens_per_expert, gbl_channel_prefix_matrix, rdma_channel_prefix_matrix,
                                 recv_gbl_rank_prefix_sum, recv_rdma_rank_prefix_sum, num_recv_tokens_per_expert,
                                 num_recv_tokens, static_cast<char *>(workspace), dev_status, stream);
    if (e != hipSuccess) return EP_ERR_HIP;
    if (num_recv_tokens_host != nullptr) {
        e = hipMemcpyAsync(num_recv_tokens_host, num_recv_tokens, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return EP_ERR_HIP;
    }
    return EP_OK;
}

ep_status_t ep_layout_notify(const ep_shape_t *s, const int64_t *topk_idx, int32_t *num_tokens_per_rank,
                             int32_t *num_tokens_per_rdma_rank, int32_t *num_tokens_per_expert,
                             uint8_t *is_token_in_rank, int32_t *gbl_channel_prefix_matrix,
                             int32_t *rdma_channel_prefix_matrix, int32_t *recv_gbl_rank_prefix_sum,
                             int32_t *recv_rdma_rank_prefix_sum, int32_t *num_recv_tokens_per_expert,
                             int32_t *num_recv_tokens, int32_t *num_recv_tokens_host, void *workspace,
                             size_t workspace_bytes, int32_t *dev_status, hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (num_tokens_per_rank == nullptr || num_tokens_per_rdma_rank == nullptr || num_tokens_per_expert == nullptr ||
        gbl_channel_prefix_matrix == nullptr || rdma_channel_prefix_matrix == nullptr ||
        recv_gbl_rank_prefix_sum == nullptr || recv_rdma_rank_prefix_sum == nullptr ||
        num_recv_tokens_per_expert == nullptr || num_recv_tokens == nullptr)
        return EP_ERR_INVALID_ARG;
    if (s->num_tokens > 0 && (topk_idx == nullptr || is_token_in_rank == nullptr)) return EP_ERR_INVALID_ARG;
    if (!workspace_ok(s, workspace, workspace_bytes)) return EP_ERR_INVALID_ARG;
    hipError_t e = launch_layout_notify(*s, topk_idx, num_tokens_per_rank, num_tokens_per_rdma_rank,
                                        num_tokens_per_expert, is_token_in_rank, gbl_channel_prefix_matrix,
                                        rdma_channel_prefix_matrix, recv_gbl_rank_prefix_sum,
                                        recv_rdma_rank_prefix_sum, num_recv_tokens_per_expert, num_recv_tokens,
                                        static_cast<char *>(workspace), dev_status, stream);
    if (e != hipSuccess) return EP_ERR_HIP;
    if (num_recv_tokens_host != nullptr) {
        e = hipMemcpyAsync(num_recv_tokens_host, num_recv_tokens, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return EP_ERR_HIP;
    }
    return EP_OK;
}

ep_status_t ep_dispatch(const ep_shape_t *s, const void *x, const int64_t *topk_idx, const float *topk_weights,
                        const uint8_t *is_token_in_rank, const int32_t *gbl_channel_prefix_matrix,
                        const int32_t *recv_gbl_rank_prefix_sum, const void *workspace, size_t workspace_bytes,
                        int32_t recv_capacity, void *recv_x, float *recv_topk_weights, int64_t *recv_topk_idx,
                        int32_t *recv_src_info, int32_t *send_slot, int32_t form, int32_t *dev_status,
                        hipStream_t stream) {
    return dispatch_checked(s, x, s ? (int64_t)s->hidden * 2 : 0, nullptr, 0, topk_idx, topk_weights,
                            is_token_in_rank, gbl_channel_prefix_matrix, recv_gbl_rank_prefix_sum, workspace,
                            workspace_bytes, recv_capacity, recv_x, nullptr, recv_topk_weights, recv_topk_idx,
                            recv_src_info, send_slot, form, dev_status, stream);
}

ep_status_t ep_dispatch_fp8(const ep_shape_t *s, const void *x, const float *x_scales, int32_t num_scales,
                            const int64_t *topk_idx, const float *topk_weights, const uint8_t *is_token_in_rank,
                            const int32_t *gbl_channel_prefix_matrix, const int32_t *recv_gbl_rank_prefix_sum,
                            const void *workspace, size_t workspace_bytes, int32_t recv_capacity, void *recv_x,
                            float *recv_x_scales, float *recv_topk_weights, int64_t *recv_topk_idx,
                            int32_t *recv_src_info, int32_t *send_slot, int32_t form, int32_t *dev_status,
                            hipStream_t stream) {
    return dispatch_checked(s, x, s ? (int64_t)s->hidden : 0, x_scales, num_scales, topk_idx, topk_weights,
                            is_token_in_rank, gbl_channel_prefix_matrix, recv_gbl_rank_prefix_sum, workspace,
                            workspace_bytes, recv_capacity, recv_x, recv_x_scales, recv_topk_weights, recv_topk_idx,
                            recv_src_info, send_slot, form, dev_status, stream);
}

ep_status_t ep_dispatch_cached(const ep_shape_t *s, const void *x, int32_t elem_bytes, const float *x_scales,
                               int32_t num_scales, const int32_t *send_slot, int32_t recv_capacity, void *recv_x,
                               float *recv_x_scales, int32_t form, int32_t *dev_status, hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (elem_bytes != 1 && elem_bytes != 2) return EP_ERR_INVALID_ARG;
    const int64_t row_bytes = (int64_t)s->hidden * elem_bytes;
    if (row_bytes % 16 != 0 || recv_capacity < 0 || !form_ok(form)) return EP_ERR_INVALID_ARG;
    if (num_scales < 0) return EP_ERR_INVALID_ARG;
    if (num_scales > kMaxScales || form == EP_FORM_PULL) return EP_ERR_UNSUPPORTED;  // cached mode: push form only
    if (s->num_tokens == 0) return EP_OK;
    if (x == nullptr || send_slot == nullptr) return EP_ERR_INVALID_ARG;
    if (recv_capacity > 0 && recv_x == nullptr) return EP_ERR_INVALID_ARG;
    if (num_scales > 0 && (x_scales == nullptr || (recv_capacity > 0 && recv_x_scales == nullptr)))
        return EP_ERR_INVALID_ARG;
    if (!aligned16(x) || (recv_x != nullptr && !aligned16(recv_x))) return EP_ERR_INVALID_ARG;
    DispatchArgs a = {};
    a.x = x;
    a.row_units = row_bytes / 16;
    a.x_scales = x_scales;
    a.num_scales = num_scales;
    a.cached_slot = send_slot;
    a.cap = recv_capacity;
    a.recv_x = recv_x;
    a.recv_scales = recv_x_scales;
    a.form = form;
    a.dev_status = dev_status;
    return from_hip(launch_dispatch(*s, a, stream));
}

ep_status_t ep_group_by_expert(const ep_shape_t *s, const void *recv_x, int32_t elem_bytes,
                               const float *recv_x_scales, int32_t num_scales, const int64_t *recv_topk_idx,
                               const float *recv_topk_weights, const int32_t *recv_gbl_rank_prefix_sum,
                               const int32_t *num_recv_tokens_per_expert, int32_t num_recv_rows,
                               int32_t grouped_capacity, void *grouped_x, float *grouped_x_scales,
                               int32_t *grouped_row, float *grouped_weights, int32_t *slot_pos,
                               int32_t *num_grouped_rows, int32_t *dev_status, hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (elem_bytes != 1 && elem_bytes != 2) return EP_ERR_INVALID_ARG;
    const int64_t row_bytes = (int64_t)s->hidden * elem_bytes;
    if (row_bytes % 16 != 0 || num_recv_rows < 0 || grouped_capacity < 0 || num_scales < 0) return EP_ERR_INVALID_ARG;
    if (num_scales > kMaxScales || s->num_experts / s->num_ranks > kMaxGroupExperts) return EP_ERR_UNSUPPORTED;
    if ((int64_t)num_recv_rows * s->num_topk > INT32_MAX) return EP_ERR_UNSUPPORTED;
    if (recv_gbl_rank_prefix_sum == nullptr || num_recv_tokens_per_expert == nullptr || num_grouped_rows == nullptr)
        return EP_ERR_INVALID_ARG;
    if (num_recv_rows > 0 && (recv_x == nullptr || recv_topk_idx == nullptr)) return EP_ERR_INVALID_ARG;
    if (grouped_capacity > 0 && (grouped_x == nullptr || grouped_row == nullptr)) return EP_ERR_INVALID_ARG;
    if (grouped_weights != nullptr && num_recv_rows > 0 && recv_topk_weights == nullptr) return EP_ERR_INVALID_ARG;
    if (num_scales > 0 && ((num_recv_rows > 0 && recv_x_scales == nullptr) ||
                           (grouped_capacity > 0 && grouped_x_scales == nullptr)))
        return EP_ERR_INVALID_ARG;
    if ((recv_x != nullptr && !aligned16(recv_x)) || (grouped_x != nullptr && !aligned16(grouped_x)))
        return EP_ERR_INVALID_ARG;
    GroupArgs a = {};
    a.recv_x = recv_x;
    a.row_units = row_bytes / 16;
    a.recv_scales = recv_x_scales;
    a.num_scales = num_scales;
    a.recv_idx = recv_topk_idx;
    a.recv_w = recv_topk_weights;
    a.recv_gbl = recv_gbl_rank_prefix_sum;
    a.aligned = num_recv_tokens_per_expert;
    a.num_rows = num_recv_rows;
    a.cap = grouped_capacity;
    a.grouped_x = grouped_x;
    a.grouped_scales = grouped_x_scales;
    a.grouped_row = grouped_row;
    a.grouped_w = grouped_weights;
    a.slot_pos = slot_pos;
    a.num_grouped = num_grouped_rows;
    a.dev_status = dev_status;
    return from_hip(launch_group(*s, a, stream));
}

ep_status_t ep_dispatch_grouped(const ep_shape_t *s, const void *x, int32_t elem_bytes, const float *x_scales,
                                int32_t num_scales, const int64_t *topk_idx, const float *topk_weights,
                                const uint8_t *is_token_in_rank, const int32_t *gbl_channel_prefix_matrix,
                                const int32_t *recv_gbl_rank_prefix_sum, const int32_t *num_recv_tokens_per_expert,
                                const void *workspace, size_t workspace_bytes, int32_t recv_capacity,
                                float *recv_topk_weights, int64_t *recv_topk_idx, int32_t *recv_src_info,
                                int32_t *send_slot, int32_t grouped_capacity, void *grouped_x,
                                float *grouped_x_scales, int32_t *grouped_row, float *grouped_weights,
                                int32_t *slot_pos, int32_t *num_grouped_rows, int32_t *dev_status,
                                hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (elem_bytes != 1 && elem_bytes != 2) return EP_ERR_INVALID_ARG;
    const int64_t row_bytes = (int64_t)s->hidden * elem_bytes;
    if (row_bytes % 16 != 0 || recv_capacity < 0 || grouped_capacity < 0 || num_scales < 0)
        return EP_ERR_INVALID_ARG;
    if (num_scales > kMaxScales || s->num_experts / s->num_ranks > kMaxGroupExperts) return EP_ERR_UNSUPPORTED;
    if ((int64_t)recv_capacity * s->num_topk > INT32_MAX) return EP_ERR_UNSUPPORTED;
    if (recv_gbl_rank_prefix_sum == nullptr || num_recv_tokens_per_expert == nullptr || num_grouped_rows == nullptr)
        return EP_ERR_INVALID_ARG;
    if (recv_capacity > 0 && (recv_topk_weights == nullptr || recv_topk_idx == nullptr || recv_src_info == nullptr ||
                              slot_pos == nullptr))
        return EP_ERR_INVALID_ARG;
    if (recv_src_info != nullptr && (reinterpret_cast<uintptr_t>(recv_src_info) & 7u) != 0) return EP_ERR_INVALID_ARG;
    if (grouped_capacity > 0 && (grouped_x == nullptr || grouped_row == nullptr)) return EP_ERR_INVALID_ARG;
    if (grouped_x != nullptr && !aligned16(grouped_x)) return EP_ERR_INVALID_ARG;
    if (num_scales > 0 && ((s->num_tokens > 0 && x_scales == nullptr) ||
                           (grouped_capacity > 0 && grouped_x_scales == nullptr)))
        return EP_ERR_INVALID_ARG;
    if (s->num_tokens > 0) {
        if (x == nullptr || topk_idx == nullptr || topk_weights == nullptr || send_slot == nullptr ||
            is_token_in_rank == nullptr || gbl_channel_prefix_matrix == nullptr)
            return EP_ERR_INVALID_ARG;
        if (!aligned16(x) || !workspace_ok(s, workspace, workspace_bytes)) return EP_ERR_INVALID_ARG;
    }
    DispatchArgs d = {};
    d.x = x;
    d.row_units = row_bytes / 16;
    d.topk_idx = topk_idx;
    d.topk_w = topk_weights;
    d.in_rank = is_token_in_rank;
    d.gbl = gbl_channel_prefix_matrix;
    d.recv_gbl = recv_gbl_rank_prefix_sum;
    d.ws = static_cast<const char *>(workspace);
    d.cap = recv_capacity;
    d.recv_w = recv_topk_weights;
    d.recv_idx = recv_topk_idx;
    d.src_info = recv_src_info;
    d.send_slot = send_slot;
    d.dev_status = dev_status;
    if (s->num_tokens > 0 && grouped_pull_applies(*s, row_bytes / 16)) {
        // one launch: routing, receive metadata, positions in token order, grouped rows, padding
        d.x_scales = x_scales;
        d.num_scales = num_scales;
        GroupedPullArgs g = {};
        g.aligned = num_recv_tokens_per_expert;
        g.cap = grouped_capacity;
        g.grouped_x = grouped_x;
        g.grouped_scales = grouped_x_scales;
        g.grouped_row = grouped_row;
        g.grouped_w = grouped_weights;
        g.slot_pos = slot_pos;
        g.num_grouped = num_grouped_rows;
        return from_hip(launch_dispatch_grouped_pull(*s, d, g, stream));
    }
    if (s->num_tokens > 0) {
        // 1. the receive metadata, with no receive rows
        hipError_t e = launch_dispatch(*s, d, stream);
        if (e != hipSuccess) return EP_ERR_HIP;
    }
    // 2. positions over the capacity's rows (rows past the last slab are not read),
    // 3. each token's row read once from x and stored at its slots' grouped positions,
    //    and the padding rows zeroed
    GroupArgs a = {};
    a.recv_x = x;
    a.from_x = true;
    a.topk_idx = topk_idx;
    a.send_slot = send_slot;
    a.num_tokens = s->num_tokens;
    a.row_units = row_bytes / 16;
    a.recv_scales = x_scales;
    a.num_scales = num_scales;
    a.recv_idx = recv_topk_idx;
    a.recv_w = recv_topk_weights;
    a.recv_gbl = recv_gbl_rank_prefix_sum;
    a.aligned = num_recv_tokens_per_expert;
    a.num_rows = recv_capacity;
    a.cap = grouped_capacity;
    a.grouped_x = grouped_x;
    a.grouped_scales = grouped_x_scales;
    a.grouped_row = grouped_row;
    a.grouped_w = grouped_weights;
    a.slot_pos = slot_pos;
    a.num_grouped = num_grouped_rows;
    a.dev_status = dev_status;
    return from_hip(launch_group(*s, a, stream));
}

ep_status_t ep_combine(const ep_shape_t *s, const void *y, const float *recv_topk_weights, const int32_t *send_slot,
                       int32_t num_recv_rows, void *combined_x, float *combined_topk_weights, int32_t *dev_status,
                       hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (num_recv_rows < 0) return EP_ERR_INVALID_ARG;
    if (s->num_tokens == 0) return EP_OK;
    if (send_slot == nullptr || combined_x == nullptr) return EP_ERR_INVALID_ARG;
    if (num_recv_rows > 0 && (y == nullptr || recv_topk_weights == nullptr)) return EP_ERR_INVALID_ARG;
    if (!aligned16(combined_x) || (y != nullptr && !aligned16(y))) return EP_ERR_INVALID_ARG;
    return from_hip(launch_combine(*s, static_cast<const uint4 *>(y), recv_topk_weights, send_slot, num_recv_rows,
                                   static_cast<uint4 *>(combined_x), combined_topk_weights, dev_status, stream));
}

ep_status_t ep_dispatch_to_fp8(const ep_shape_t *s, const void *x, int32_t num_scales, const int64_t *topk_idx,
                              const float *topk_weights, const uint8_t *is_token_in_rank,
                              const int32_t *gbl_channel_prefix_matrix, const int32_t *recv_gbl_rank_prefix_sum,
                              const void *workspace, size_t workspace_bytes, int32_t recv_capacity, void *recv_x,
                              float *recv_x_scales, float *recv_topk_weights, int64_t *recv_topk_idx,
                              int32_t *recv_src_info, int32_t *send_slot, int32_t *dev_status, hipStream_t stream) {
    const ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (s->hidden % kQuantChannels != 0 || num_scales < 1 || s->hidden % num_scales != 0) return EP_ERR_INVALID_ARG;
    const int l = quant_lanes_log2(s->hidden, num_scales);
    if (l < 0) return EP_ERR_UNSUPPORTED;
    return dispatch_checked(s, x, (int64_t)s->hidden, nullptr, num_scales, topk_idx, topk_weights, is_token_in_rank,
                            gbl_channel_prefix_matrix, recv_gbl_rank_prefix_sum, workspace, workspace_bytes,
                            recv_capacity, recv_x, recv_x_scales, recv_topk_weights, recv_topk_idx, recv_src_info,
                            send_slot, EP_FORM_PUSH, dev_status, stream, l);
}

ep_status_t ep_dispatch_cached_to_fp8(const ep_shape_t *s, const void *x, int32_t num_scales, const int32_t *send_slot,
                                     int32_t recv_capacity, void *recv_x, float *recv_x_scales, int32_t *dev_status,
                                     hipStream_t stream) {
    ep_status_t st = check_shape(s);
    if (st != EP_OK) return st;
    if (s->hidden % kQuantChannels != 0 || num_scales < 1 || s->hidden % num_scales != 0 || recv_capacity < 0)
        return EP_ERR_INVALID_ARG;
    const int l = quant_lanes_log2(s->hidden, num_scales);
    if (l < 0 || num_scales > kMaxScales) return EP_ERR_UNSUPPORTED;
    if (s->num_tokens == 0) return EP_OK;
    if (x == nullptr || send_slot == nullptr) return EP_ERR_INVALID_ARG;
    if (recv_capacity > 0 && (recv_x == nullptr || recv_x_scales == nullptr)) return EP_ERR_INVALID_ARG;
    if (!aligned16(x) || (recv_x != nullptr && !aligned16(recv_x))) return EP_ERR_INVALID_ARG;
    DispatchArgs a = {};
    a.x = x;
    a.row_units = s->hidden / 16;  // units of the fp8 row
    a.x_scales = nullptr;
    a.num_scales = num_scales;
    a.cached_slot = send_slot;
    a.cap = recv_capacity;
    a.recv_x = recv_x;
    a.recv_scales = recv_x_scales;
    a.form = EP_FORM_PUSH;
    a.dev_status = dev_status;
    a.quantize = true;
    a.quant_log2 = l;
    return from_hip(launch_dispatch(*s, a, stream));
}

ep_status_t ep_quantize_fp8(const void *x, int64_t num_rows, int32_t hidden, int32_t num_scales, void *x_fp8,
                            float *x_scales, hipStream_t stream) {
    const ep_status_t st = quant_checked(x, x_fp8, x_scales, num_rows, hidden, num_scales);
    if (st != EP_OK || num_rows == 0) return st;
    return from_hip(launch_quantize(x, num_rows, hidden, num_scales, x_fp8, x_scales, stream));
}

ep_status_t ep_dequantize_fp8(const void *x_fp8, const float *x_scales, int64_t num_rows, int32_t hidden,
                              int32_t num_scales, void *out, hipStream_t stream) {
    const ep_status_t st = quant_checked(out, x_fp8, x_scales, num_rows, hidden, num_scales);
    if (st != EP_OK || num_rows == 0) return st;
    return from_hip(launch_dequantize(x_fp8, x_scales, num_rows, hidden, num_scales, out, stream));
}

}  // extern "C"
