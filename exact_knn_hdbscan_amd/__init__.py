"""Exact kNN, HDBSCAN core distances, Boruvka MST and the HDBSCAN tail on MI355X (gfx950).

The compute lives in the HIP library ``libekh.so`` (C ABI declared in
``include/ekh.h``); ``exact_knn_hdbscan_amd.binding`` marshals torch tensors
to it.  The binding is loaded on first use of one of the entry points below so
that ``exact_knn_hdbscan_amd.datagen`` can be imported without a GPU.
"""
_ENTRY_POINTS = ("knn", "knn_noalloc", "core_distances", "mst_boruvka", "knn_workspace_bytes", "knn_plan", "core_workspace_bytes",
                 "mst_workspace_bytes", "hdbscan_tail", "bipartite_assign", "bipartite_workspace_bytes",
                 "cluster_edge_counts", "merge_tree", "kmeanspp", "kmeanspp_workspace_bytes", "library", "MstStats", "EkhError", "kernel_timer")

__all__ = list(_ENTRY_POINTS)


def __getattr__(name):
    if name in _ENTRY_POINTS:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
