/*
 * pa_probe.h -- measurement helper of libpa.so: the achievable HBM read
 * bandwidth the decode kernels' roofline is read against.
 *
 * The decode path is bound by reading the KV cache from HBM ("Inside vLLM"
 * §3.3: decode reads the cached history; "vllm v1 源码精读（三）" §4.2: decode
 * is memory-bandwidth bound), so its fraction of the chip's published HBM
 * peak is set next to what a plain streaming read reaches on the same part.
 * Not part of the attention path.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_read_probe -- stream `bytes` of device memory at `src` through the
 * vector load units and discard them: each work-group of 4 wavefronts reads
 * one contiguous slice, every lane 16 bytes per load with 8 loads in flight,
 * so each load instruction of a wavefront covers 1 KiB of consecutive bytes.
 * The loads carry the non-temporal hint, as the decode kernels' K/V loads do
 * (data read once).
 * The grid holds `waves_per_simd` wavefronts per SIMD of the device (1, 2 or
 * 4; the CU count is read from the device).  `sink` (device, 4 bytes) is
 * written only when a checksum of the data equals a value no buffer
 * produces in practice: the loads cannot be removed, and nothing else is
 * written.  src and bytes must be multiples of 16.  Asynchronous on `stream`;
 * returns a pa_status (PA_ERR_INVALID_ARG for bad arguments).
 */
int pa_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t waves_per_simd,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
