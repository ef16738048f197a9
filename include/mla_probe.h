/*
 * Read-bandwidth probes (libmla_probe.so): measurement support for the roofline of
 * MLA decode, not part of the decode path.  The main kernel is bound by HBM reads;
 * these calls measure what reads alone reach on the device, in two shapes:
 *
 *   mla_probe_stream_read  reads `bytes` (a multiple of 16) of `buf` with 16-byte loads
 *                          in a grid-stride loop, eight in flight per thread, over
 *                          `workgroups` workgroups of 256 threads; nontemporal != 0 adds
 *                          the non-temporal hint to every load.
 *   mla_probe_page_read    the decode's page-copy structure without its compute: one
 *                          workgroup of 4 waves per compute unit (`workgroups` of them)
 *                          walks its share of order[0 .. nunits) (contiguous shares, in
 *                          list order), copying block order[k] (unit_bytes bytes at
 *                          buf + order[k] * unit_bytes) into LDS with 16-byte
 *                          direct-to-LDS loads, nbuf LDS buffers (nbuf - 1 blocks in
 *                          flight).  (unit_bytes, nbuf) is one of (73728, 2) (a 64-token
 *                          page, two buffers as in the main kernel), (36864, 3),
 *                          (36864, 4) or (16384, 8); else -2.
 *
 * buf, order, sink: device pointers.  buf is 16-byte aligned; every order[k] must name a
 * block inside buf (the caller checks: it is not checked on the device).  sink: device
 * scratch of workgroups * 256 uint32, written only on a data pattern that does not occur
 * (it keeps the loads from being removed).  Returns 0, -1 (bad argument), -2 (unsupported
 * shape) or -4 (launch failed).  Asynchronous on `stream` (a hipStream_t).
 */
#ifndef MLA_PROBE_H
#define MLA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int mla_probe_stream_read(const void* buf, size_t bytes, int nontemporal, int workgroups,
                          uint32_t* sink, void* stream);
int mla_probe_page_read(const void* buf, int unit_bytes, int nbuf, const int32_t* order,
                        int nunits, int workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROBE_H */
