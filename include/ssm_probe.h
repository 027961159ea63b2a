/* Measurement probes for the roofline model of the scan kernels (gfx950).
 *
 * Not part of the scan's interface: a separate library, libssm_probe.so,
 * that the benchmark harness loads to measure, on the device it runs on, the
 * rates its VALU roofline assumes. The scan's transition needs one
 * exponential per state update (the e^(dt A) of the discretisation,
 * "从 Transformer 到 Mamba", ybb.press, section 3.1), so the bound of the scan
 * is the vector ALU's issue rate of v_exp_f32 next to the FMA-pipe ops, which
 * no vendor table gives.
 *
 * Every rate is in lane operations per second over the whole device, from
 * HIP events around launches of register-only kernels (no memory traffic
 * beyond one store per thread) that fill every SIMD with eight waves:
 *   exp_lanes_per_s   chains of v_exp_f32
 *   fma_lanes_per_s   chains of v_fma_f32
 *   mix_slots_per_s   the scan's per-update mix (two multiplies, one
 *                     v_exp_f32, two FMAs), counted as 6 slots per update
 *                     (the exponential as 2): the model's peak is reached
 *                     when this equals 64 slots per clock per CU
 *   mix2_slots_per_s  the same mix at two waves per SIMD (one block of eight
 *                     waves per CU), the occupancy of the scan at N = 16
 *   copy_bytes_per_s  a streaming device copy (bytes read + written), 1 GiB
 * cus and clock_khz are the device's compute-unit count and peak engine clock
 * as the runtime reports them.
 *
 * Ownership and errors: the call allocates and frees its own device buffers
 * (it is a measurement tool, not a hot path), synchronises the device, and
 * returns 0, or the HIP error code of the first failing call.
 */
#ifndef SSM_PROBE_H
#define SSM_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  double exp_lanes_per_s;
  double fma_lanes_per_s;
  double mix_slots_per_s;
  double mix2_slots_per_s;
  double copy_bytes_per_s;
  int cus;
  int clock_khz;
} ssm_probe_rates_t;

/* Runs the probes on the current device. `out` is a host pointer. */
int ssm_probe_valu(ssm_probe_rates_t* out);

#ifdef __cplusplus
}
#endif

#endif /* SSM_PROBE_H */
