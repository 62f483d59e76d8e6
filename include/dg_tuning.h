/*
 * dg_tuning.h -- tuning and introspection hooks of libdg.so.  NOT part of the
 * library's contract (dg.h): they exist so that tests can run every compiled tile
 * configuration against the others and so that a launch plan can be inspected
 * without running it.  They may change with the set of compiled kernels.
 */
#ifndef DG_TUNING_H
#define DG_TUNING_H

#ifdef __cplusplus
extern "C" {
#endif

/* Pin the kernel configuration (an id reported by dg_describe_launch) for every
 * later call of that configuration's layout, overriding the planner; -1 restores
 * automatic planning for all layouts.  Meant for tuning and for tests that
 * compare tile shapes.  Unknown ids give DG_ERR_INVALID_ARG.  The setting belongs to
 * the calling thread: calls made from other threads keep planning on their own. */
int dg_set_kernel_config(int config_id);

/* Enumerate the compiled kernel configurations: for index 0, 1, ... fills
 * out[0..7] = config id, layout, block_m, block_n, waves per workgroup, 1 if
 * the configuration also runs E5M2 operands (the _fmt calls) else 0, 1 if it
 * has instances compiled for fixed N and K (see dg_describe_launch) else 0, and
 * the number of K groups (1; 2 where two groups of waves each sum every other K
 * block of a tile and the two sums are added at the end, which rounds differently
 * from one chain over all K blocks), and returns DG_OK; past the last one returns
 * DG_ERR_INVALID_ARG.  out must hold 8 ints.  Host only. */
int dg_kernel_config_info(int index, int* out);

/* Describe the kernel configuration a call with these sizes would launch, without
 * launching (layout 0 dense, 1 contiguous, 2 masked).  out[0..7] = block_m,
 * block_n, waves per workgroup, tiles (upper bound for masked), persistent grid
 * size, config id, row tiles per raster group of the tile order (0 for masked,
 * whose order follows the groups), and K/128 if the launch uses an instance
 * compiled for this N and K (in some configurations: dense N = 7168 with K = 7168
 * or 2048, contiguous and masked N = 4096 with K = 7168), else 0; out must hold 8
 * ints.  num_cus <= 0 uses
 * dg_get_num_cus().  Needs no device if num_cus > 0 and assumes one resident
 * workgroup per CU for the big shapes. */
int dg_describe_launch(int layout, int m, int n, int k, int num_groups, int num_cus, int* out);

#ifdef __cplusplus
}
#endif

#endif /* DG_TUNING_H */
