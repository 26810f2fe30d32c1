/* kvc_probe.h — HBM read probes of the kvc library (MI355X, gfx950): measurement utilities, not part of the
 * compressed-KV method. They give a ceiling and a floor to compare the decode kernels with: how fast this GPU
 * streams reads from HBM, and how long one launch takes just to load a given number of bytes in the per-wave
 * pattern the decode kernel uses.
 *
 * Both read `bytes` of `buf` (device memory, 16-byte aligned, bytes a multiple of 16) with 16-byte vector loads and
 * fold what they read into one 32-bit word per workgroup, written to sink[workgroup] (so no load can be dropped);
 * the sink's contents are meaningless. Asynchronous on `stream`; return 0 (KVC_OK) or a negative kvc_status. */
#ifndef KVC_PROBE_H_
#define KVC_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: `workgroups` workgroups of 256 threads (0: eight per compute unit) walk the buffer with a
 * grid-wide stride, eight 16-byte loads in flight per thread. sink: [workgroups] uint32 (query with
 * kvc_probe_stream_workgroups). bytes <= 2^40. */
int kvc_probe_stream_workgroups(int32_t workgroups);
int kvc_probe_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream);

/* Per-wave read, the decode kernel's pattern for a full-precision window: every wave loads one contiguous 16 KiB
 * task (sixteen 16-byte loads per lane, all issued before the first use), eight waves per workgroup. Tasks are
 * bytes / 16384 (bytes a multiple of 16384, at most 2^36); sink: [ceil(tasks / 8)] uint32. */
int kvc_probe_wave_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_PROBE_H_ */
