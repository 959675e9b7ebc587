// wkv_workspace_errors: whether the one-launch split calls on a workspace kept
// their results.  A bounded wait of the one launch that expires marks the
// error word of its (sequence, head) control record (SplitCtl), and that
// call's results are void; the kernels only ever set that word, so it stays
// until a caller clears it here.  A call whose wait expired can also leave
// the record's counters out of step (a late arrival counted after the record
// was reset for the next call), which a later call would read as an arrival
// of its own; clearing therefore zeroes the whole record, the state every
// record starts from.  Without an expired wait every count of a call lands
// before its last main workgroup resets the record, so unmarked records are
// left as they are.
#include <cstdio>
#include <vector>

#include "wkv_internal.h"

extern "C" wkv_status_t wkv_workspace_errors(const void *workspace, size_t workspace_bytes, int clear,
                                             int *count, void *stream) {
    using namespace finch;
    record_error(WKV_OK, "");                   // no detail left from an earlier call
    if (!count) return record_error(WKV_EINVAL, "count is NULL");
    *count = 0;
    const char *base = static_cast<const char *>(workspace);
    if (!base) {
        base = static_cast<const char *>(static_scratch_if_set());
        if (!base) return WKV_OK;               // no allocation-free call on this device yet
    } else if (workspace_bytes == 0) {
        return WKV_OK;                          // a call that needed no workspace: no records
    } else if (workspace_bytes < (size_t)WKV_WORKSPACE_CONTROL_BYTES) {
        char msg[160];
        snprintf(msg, sizeof msg, "workspace_bytes=%zu is below the %d bytes of control records",
                 workspace_bytes, WKV_WORKSPACE_CONTROL_BYTES);
        return record_error(WKV_EWORKSPACE, msg);
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    std::vector<SplitCtl> rec(kCtlRecords);
    hipError_t e = hipMemcpyAsync(rec.data(), base, WKV_WORKSPACE_CONTROL_BYTES, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return record_error(WKV_EHIP, hipGetErrorString(e));
    int marked = 0;
    for (int i = 0; i < kCtlRecords; ++i) {
        if (rec[i].error == 0) continue;
        ++marked;
        if (clear) {
            char *at = const_cast<char *>(base) + i * sizeof(SplitCtl);
            if ((e = hipMemsetAsync(at, 0, sizeof(SplitCtl), st)) != hipSuccess)
                return record_error(WKV_EHIP, hipGetErrorString(e));
        }
    }
    if (clear && marked > 0 && (e = hipStreamSynchronize(st)) != hipSuccess)
        return record_error(WKV_EHIP, hipGetErrorString(e));
    *count = marked;
    return WKV_OK;
}
